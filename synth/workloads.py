"""Named MLA decode workloads and their seeded synthetic inputs.

Shapes follow the DeepSeek-V2 geometry (DeepSeek V2 MLA page, section 3.1:
128 heads, head dim 128, latent d_c = 512, decoupled RoPE d_r = 64).  Values:
q_C, q_R, c_KV, k_R ~ N(0, 1); W_UK, W_UV ~ N(0, 1/d_c).

Stream ids under one base seed: 0 q_C, 1 q_R, 2 c_KV, 3 k_R, 4 W_UK, 5 W_UV,
6 ragged lengths, 7 page permutation.  Cache element d of token t of sequence b
is counter (b * 2^24 + t) * width + d of its stream, so the contiguous and the
paged layouts hold the same values for the same (b, t), and a long cache can be
regenerated one sequence at a time.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional, Sequence

import numpy as np

from .encode import f32_to_bf16_bits, quantize_rows_e4m3, round_to_f32
from .rng import permutation, randint_uniform, standard_normal

BASE_SEED = 0x4D4C41
TOKEN_STRIDE = 1 << 24  # counter stride between sequences (max tokens per sequence)

S_QNOPE, S_QROPE, S_LATENT, S_KROPE, S_WUK, S_WUV, S_LENS, S_PERM = range(8)

# bit patterns used to fill cache slots that must never be read
NAN_BF16 = np.uint16(0x7FC0)
NAN_E4M3 = np.uint8(0x7F)


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int = 128
    d_nope: int = 128
    d_rope: int = 64
    d_latent: int = 512
    d_v: int = 128
    cache_dtype: str = "bf16"  # "f32" | "bf16" | "fp8"
    act_dtype: str = "bf16"  # dtype of q_C, q_R, W_UK, W_UV: "f32" | "bf16"
    out_dtype: str = "bf16"  # dtype of o
    seq_len: Optional[int] = 2048  # uniform length; None = ragged
    len_range: Optional[tuple] = None  # inclusive (lo, hi) of ragged lengths
    page_size: int = 0  # 0 = contiguous rows, else tokens per page
    num_splits: int = 1
    # "fixed": mla_decode's split ranges; "balanced": the decode's balanced
    # partition of the batch (mla_decode_ex, MLA_KERNEL_H64_BALANCED), with
    # at most num_splits pieces per sequence
    partition: str = "fixed"
    seed: int = BASE_SEED
    description: str = ""

    @property
    def row_width(self) -> int:
        return self.d_latent + self.d_rope

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.d_nope + self.d_rope)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny_f32": Workload(
        "tiny_f32", batch=1, heads=16, cache_dtype="f32", act_dtype="f32",
        out_dtype="f32", seq_len=512, num_splits=1, seed=BASE_SEED + 1,
        description="tiny fp32 decode: B=1, h=16, L=512"),
    "dsv2_b32_l2k": Workload(
        "dsv2_b32_l2k", batch=32, seq_len=2048, num_splits=4, seed=BASE_SEED + 2,
        description="DeepSeek-V2 geometry bf16 decode: B=32, h=128, L=2048"),
    "long_b4_l32k": Workload(
        "long_b4_l32k", batch=4, seq_len=32768, num_splits=64, seed=BASE_SEED + 3,
        description="long-context bf16 decode: B=4, L=32768, 64 splits"),
    "paged_b64_ragged": Workload(
        "paged_b64_ragged", batch=64, seq_len=None, len_range=(512, 16384),
        page_size=64, num_splits=5, partition="balanced", seed=BASE_SEED + 4,
        description="paged ragged bf16 decode: B=64, L~U[512,16384], 64-token pages; "
                    "balanced partition, at most 5 splits per sequence"),
    "fp8_b1_l128k": Workload(
        "fp8_b1_l128k", batch=1, seq_len=131072, cache_dtype="fp8", num_splits=256,
        seed=BASE_SEED + 5,
        description="128K fp8-e4m3 cache decode: B=1, L=131072, 256 splits"),
    "fp8_b8_l128k": Workload(
        "fp8_b8_l128k", batch=8, seq_len=131072, cache_dtype="fp8", num_splits=256,
        seed=BASE_SEED + 5,
        description="128K fp8-e4m3 cache decode: B=8, L=131072, 256 splits"),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


@dataclass
class MLAInputs:
    """Stored (bit-level) inputs of one decode step.

    Array dtypes: float32 for "f32", uint16 bit patterns for "bf16",
    uint8 codes for "fp8".
    """

    wl: Workload
    q_nope: np.ndarray  # [B, h, d_nope]
    q_rope: np.ndarray  # [B, h, d_rope]
    w_uk: np.ndarray  # [h, d_nope, d_latent]
    w_uv: np.ndarray  # [h, d_v, d_latent]
    rows: np.ndarray  # [n_rows, d_latent + d_rope]
    row_scale: Optional[np.ndarray]  # float32 [n_rows] (fp8 only)
    seq_lens: np.ndarray  # int32 [B]
    seq_stride: int  # contiguous: rows between sequences
    block_table: Optional[np.ndarray]  # int32 [B, max_pages] (paged)
    max_seq_len: int

    @property
    def max_pages(self) -> int:
        return 0 if self.block_table is None else int(self.block_table.shape[1])

    def row_index(self, b: int, t: int) -> int:
        """Physical row holding token t of sequence b."""
        if self.wl.page_size:
            ps = self.wl.page_size
            return int(self.block_table[b, t // ps]) * ps + t % ps
        return b * self.seq_stride + t


def _store(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = round_to_f32(x64)
    if dtype == "f32":
        return x32
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    raise ValueError(dtype)


def _nan_fill(dtype: str):
    return {"f32": np.float32(np.nan), "bf16": NAN_BF16, "fp8": NAN_E4M3}[dtype]


def _storage_dtype(dtype: str):
    return {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}[dtype]


def sequence_lengths(wl: Workload) -> np.ndarray:
    if wl.seq_len is not None:
        return np.full(wl.batch, wl.seq_len, dtype=np.int32)
    lo, hi = wl.len_range
    return randint_uniform(wl.seed, S_LENS, lo, hi, wl.batch).astype(np.int32)


def token_rows(wl: Workload, b: int, t0: int, n: int) -> np.ndarray:
    """float32 [n, d_latent + d_rope] values of tokens t0..t0+n-1 of sequence b
    (before any fp8 quantization)."""
    w = wl.row_width
    base = b * TOKEN_STRIDE + t0
    lat = standard_normal(wl.seed, S_LATENT, base * wl.d_latent, n * wl.d_latent)
    rope = standard_normal(wl.seed, S_KROPE, base * wl.d_rope, n * wl.d_rope)
    out = np.empty((n, w), dtype=np.float32)
    out[:, : wl.d_latent] = round_to_f32(lat).reshape(n, wl.d_latent)
    out[:, wl.d_latent:] = round_to_f32(rope).reshape(n, wl.d_rope)
    return out


def _encode_rows(wl: Workload, vals32: np.ndarray):
    if wl.cache_dtype == "f32":
        return vals32, None
    if wl.cache_dtype == "bf16":
        return f32_to_bf16_bits(vals32), None
    if wl.cache_dtype == "fp8":
        return quantize_rows_e4m3(vals32)
    raise ValueError(wl.cache_dtype)


def make_inputs(wl: Workload, lengths: Optional[Sequence[int]] = None,
                seq_stride: Optional[int] = None, poison: bool = True) -> MLAInputs:
    """Build the stored inputs of a workload.

    lengths overrides the per-sequence lengths (ragged tests).  Cache slots that
    belong to no token (past a sequence's length in the contiguous layout, the
    tail of a sequence's last page in the paged layout) hold NaN bit patterns
    when poison is set, so that a reader of unowned slots is caught.
    """
    B, h = wl.batch, wl.heads
    seq_lens = (np.asarray(lengths, dtype=np.int32) if lengths is not None
                else sequence_lengths(wl))
    assert seq_lens.shape == (B,)
    max_len = int(seq_lens.max()) if B else 0

    q_nope = _store(standard_normal(wl.seed, S_QNOPE, 0, B * h * wl.d_nope), wl.act_dtype)
    q_rope = _store(standard_normal(wl.seed, S_QROPE, 0, B * h * wl.d_rope), wl.act_dtype)
    wstd = 1.0 / math.sqrt(wl.d_latent)
    w_uk = _store(standard_normal(wl.seed, S_WUK, 0, h * wl.d_nope * wl.d_latent) * wstd,
                  wl.act_dtype)
    w_uv = _store(standard_normal(wl.seed, S_WUV, 0, h * wl.d_v * wl.d_latent) * wstd,
                  wl.act_dtype)

    W = wl.row_width
    sdt = _storage_dtype(wl.cache_dtype)
    fp8 = wl.cache_dtype == "fp8"
    block_table = None
    if wl.page_size:
        ps = wl.page_size
        npages = [(int(L) + ps - 1) // ps for L in seq_lens]
        total = int(sum(npages))
        perm = permutation(wl.seed, S_PERM, total)
        maxp = max(npages) if npages else 0
        block_table = np.full((B, max(maxp, 1)), -1, dtype=np.int32)
        n_rows = total * ps
        stride = 0
    else:
        stride = int(seq_stride) if seq_stride is not None else max_len
        assert stride >= max_len
        n_rows = B * stride
    rows = np.empty((n_rows, W), dtype=sdt)
    rows[...] = _nan_fill(wl.cache_dtype) if poison else 0
    row_scale = None
    if fp8:
        row_scale = np.full(n_rows, np.nan if poison else 0.0, dtype=np.float32)

    g = 0
    for b in range(B):
        L = int(seq_lens[b])
        if L == 0:
            continue
        enc, sc = _encode_rows(wl, token_rows(wl, b, 0, L))
        if wl.page_size:
            ps = wl.page_size
            for j in range((L + ps - 1) // ps):
                phys = int(perm[g])
                g += 1
                block_table[b, j] = phys
                n = min(ps, L - j * ps)
                rows[phys * ps: phys * ps + n] = enc[j * ps: j * ps + n]
                if fp8:
                    row_scale[phys * ps: phys * ps + n] = sc[j * ps: j * ps + n]
        else:
            rows[b * stride: b * stride + L] = enc
            if fp8:
                row_scale[b * stride: b * stride + L] = sc

    return MLAInputs(wl=wl, q_nope=q_nope.reshape(B, h, wl.d_nope),
                     q_rope=q_rope.reshape(B, h, wl.d_rope),
                     w_uk=w_uk.reshape(h, wl.d_nope, wl.d_latent),
                     w_uv=w_uv.reshape(h, wl.d_v, wl.d_latent),
                     rows=rows, row_scale=row_scale, seq_lens=seq_lens,
                     seq_stride=stride, block_table=block_table, max_seq_len=max_len)


def cache_bytes(wl: Workload, seq_lens: np.ndarray) -> int:
    """Bytes of latent cache one decode step must read: sum_b L_b * row bytes
    (+4 bytes of row scale for fp8)."""
    per = wl.row_width * {"f32": 4, "bf16": 2, "fp8": 1}[wl.cache_dtype]
    if wl.cache_dtype == "fp8":
        per += 4
    return int(np.sum(seq_lens.astype(np.int64))) * per

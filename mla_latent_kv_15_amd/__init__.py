"""Python binding of libmla.so, the MI355X (gfx950) MLA decode library.

Argument marshalling only: every function here takes torch tensors that live
on the GPU, checks their device, dtype, exact shape (from the batch, split
count, heads and widths the call implies) and contiguity before anything
reaches the library, and passes raw device
pointers plus the current HIP stream to the C entry point of the same name
declared in include/mla.h.  All arithmetic runs in the library's kernels.
There is no CPU fallback: importing this module without the built library
raises.
"""

from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla.so")

MLA_F32, MLA_BF16, MLA_FP8_E4M3 = 0, 1, 2
MLA_OK = 0

D_LATENT = 512
D_ROPE = 64
TILE_TOKENS = 32
PAGE_SIZE = 64
MAX_SPLITS = 1024


class MLAError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {status_str(status)} (status {status})")
        self.status = status


class Dims(C.Structure):
    _fields_ = [("heads", C.c_int32), ("d_nope", C.c_int32), ("d_rope", C.c_int32),
                ("d_latent", C.c_int32), ("d_v", C.c_int32), ("softmax_scale", C.c_float)]


class CacheDesc(C.Structure):
    _fields_ = [("dtype", C.c_int32), ("rows", C.c_void_p), ("row_scale", C.c_void_p),
                ("page_size", C.c_int32), ("seq_stride", C.c_int64),
                ("block_table", C.c_void_p), ("max_pages", C.c_int32),
                ("seq_lens", C.c_void_p), ("max_seq_len", C.c_int32), ("ring", C.c_int32)]


_lib = None


def lib():
    """The loaded libmla.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = C.CDLL(LIB_PATH)
        vp, i32, f32p = C.c_void_p, C.c_int32, C.c_void_p
        L.mla_absorb_q.restype = C.c_int
        L.mla_absorb_q.argtypes = [C.POINTER(Dims), i32, vp, vp, i32, vp, i32, vp, i32, f32p, vp]
        L.mla_decode.restype = C.c_int
        L.mla_decode.argtypes = [C.POINTER(Dims), i32, vp, i32, f32p, C.POINTER(CacheDesc), i32,
                                 vp, i32, f32p, vp]
        L.mla_decode_ex.restype = C.c_int
        L.mla_decode_ex.argtypes = [C.POINTER(Dims), i32, i32, vp, i32, C.POINTER(CacheDesc), i32,
                                    vp, i32, f32p, i32, vp]
        L.mla_decode_multi.restype = C.c_int
        L.mla_decode_multi.argtypes = [C.POINTER(Dims), i32, i32, vp, i32, C.POINTER(CacheDesc),
                                       i32, vp, i32, f32p, vp]
        L.mla_combine.restype = C.c_int
        L.mla_combine.argtypes = [C.POINTER(Dims), i32, i32, vp, i32, f32p, vp, i32, f32p, vp]
        L.mla_up_proj.restype = C.c_int
        L.mla_up_proj.argtypes = [C.POINTER(Dims), i32, vp, i32, vp, i32, vp, i32, vp]
        L.mla_combine_up_proj.restype = C.c_int
        L.mla_combine_up_proj.argtypes = [C.POINTER(Dims), i32, i32, vp, i32, f32p, vp, i32, vp,
                                          i32, vp, f32p, vp]
        L.mla_absorb_q_rope.restype = C.c_int
        L.mla_absorb_q_rope.argtypes = [C.POINTER(Dims), i32, vp, vp, i32, vp, i32, vp,
                                        C.c_float, vp, i32, vp]
        L.mla_mha_decode.restype = C.c_int
        L.mla_mha_decode.argtypes = [i32, i32, i32, vp, vp, vp, i32, vp, C.c_int64, i32,
                                     C.c_float, vp, i32, f32p, vp]
        L.mla_gqa_decode.restype = C.c_int
        L.mla_gqa_decode.argtypes = [i32, i32, i32, i32, vp, vp, vp, i32, vp, C.c_int64, i32,
                                     C.c_float, vp, i32, f32p, vp]
        L.mla_cache_append.restype = C.c_int
        L.mla_cache_append.argtypes = [C.POINTER(Dims), i32, vp, vp, i32, vp,
                                       C.POINTER(CacheDesc), vp]
        L.mla_decode_combine_up_proj_noalloc.restype = C.c_int
        L.mla_decode_combine_up_proj_noalloc.argtypes = [C.POINTER(Dims), i32, vp, i32,
                                                         C.POINTER(CacheDesc), i32, vp, i32, vp,
                                                         i32, vp, f32p, vp]
        L.mla_cache_ring_grow.restype = C.c_int
        L.mla_cache_ring_grow.argtypes = [i32, C.POINTER(CacheDesc), C.POINTER(CacheDesc), vp]
        L.mla_prefill_rebuild_kv.restype = C.c_int
        L.mla_prefill_rebuild_kv.argtypes = [C.POINTER(Dims), i32, C.POINTER(CacheDesc), vp, vp, vp,
                                             i32, vp, vp, C.c_int64, vp]
        L.mla_prefill_attn.restype = C.c_int
        L.mla_prefill_attn.argtypes = [C.POINTER(Dims), i32, i32, vp, vp, i32, vp, vp, C.c_int64,
                                       vp, i32, vp, i32, f32p, vp]
        L.mla_stream_probe.restype = C.c_int
        L.mla_stream_probe.argtypes = [vp, C.c_int64, i32, i32, i32, vp, vp]
        L.mla_status_str.restype = C.c_char_p
        L.mla_status_str.argtypes = [C.c_int]
        L.mla_version.restype = C.c_int32
        L.mla_version.argtypes = []
        _lib = L
    return _lib


EXPORTED = ("mla_absorb_q", "mla_decode", "mla_decode_multi", "mla_decode_ex", "mla_combine", "mla_up_proj", "mla_combine_up_proj",
            "mla_absorb_q_rope", "mla_cache_append", "mla_mha_decode", "mla_status_str",
            "mla_version", "mla_decode_combine_up_proj_noalloc", "mla_cache_ring_grow",
            "mla_gqa_decode", "mla_prefill_rebuild_kv", "mla_prefill_attn", "mla_stream_probe")


def status_str(status: int) -> str:
    return lib().mla_status_str(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != MLA_OK:
        raise MLAError(fn, status)


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MLA_F32
    if t.dtype == torch.bfloat16:
        return MLA_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return MLA_FP8_E4M3
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the MLA library must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"tensors passed to the MLA library must be on the GPU, got {t.device}")
    return t.data_ptr()


def _need(name: str, t: Optional[torch.Tensor], shape, dtypes=None, optional=False) -> None:
    """Checks, before anything reaches the C library, that `t` is a tensor of
    exactly `shape` (and of one of `dtypes`) and contiguous: the
    kernels index every buffer by the sizes the call implies, so a smaller
    buffer would be read or written out of bounds."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    shape = tuple(int(x) for x in shape)
    if tuple(t.shape) != shape:
        raise ValueError(f"{name} has shape {tuple(t.shape)}, the call needs {shape}")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, the call needs one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on_gpu(*ts) -> None:
    """every given buffer (None: absent) lives on the GPU; checked after the
    shapes, so a shape error is reported as such whatever the device"""
    for x in ts:
        if x is not None and x.device.type != "cuda":
            raise ValueError(f"tensors passed to the MLA library must be on the GPU, got {x.device}")


def _cache_tensors(cache: "Cache"):
    return (cache.rows, cache.seq_lens, cache.row_scale, cache.block_table)


_FLOAT = (torch.float32, torch.bfloat16)
_CACHE_DT = (torch.float32, torch.bfloat16, torch.uint8, torch.float8_e4m3fn)


def _need_cache(cache: "Cache", B: int, geo: "Geometry") -> None:
    """The cache descriptor's buffers against the batch: rows [n, 576],
    seq_lens int32 [B], block_table int32 [B, max_pages] (paged), row_scale
    float32 [n] (e4m3); a contiguous cache must hold B * seq_stride rows (the
    last sequence at least max_seq_len).  Page ids inside block_table live on
    the device and are the caller's contract."""
    w = geo.d_latent + geo.d_rope
    r = cache.rows
    if not isinstance(r, torch.Tensor) or r.dim() != 2 or int(r.shape[1]) != w:
        raise ValueError(f"cache.rows must be [n_rows, {w}]")
    _need("cache.rows", r, tuple(r.shape), _CACHE_DT)
    n = int(r.shape[0])
    _need("cache.seq_lens", cache.seq_lens, (B,), (torch.int32,))
    if int(cache.max_seq_len) < 0:
        raise ValueError("cache.max_seq_len must be >= 0")
    if dtype_code(r) == MLA_FP8_E4M3:
        _need("cache.row_scale", cache.row_scale, (n,), (torch.float32,))
    if cache.ring:
        if cache.page_size:
            raise ValueError("a ring cache is contiguous (page_size 0)")
        if int(cache.seq_stride) < 1 or B * int(cache.seq_stride) > n:
            raise ValueError(f"cache.rows holds {n} rows, B={B} rings of {cache.seq_stride} "
                             f"need {B * cache.seq_stride}")
    elif cache.page_size:
        bt = cache.block_table
        if not isinstance(bt, torch.Tensor) or bt.dim() != 2:
            raise ValueError("a paged cache needs block_table [B, max_pages]")
        _need("cache.block_table", bt, (B, int(bt.shape[1])), (torch.int32,))
        if int(bt.shape[1]) * int(cache.page_size) < int(cache.max_seq_len):
            raise ValueError("block_table has fewer pages than max_seq_len needs")
    elif B > 0 and cache.max_seq_len > 0:
        if int(cache.seq_stride) < int(cache.max_seq_len):
            raise ValueError("cache.seq_stride must be >= max_seq_len")
        if (B - 1) * int(cache.seq_stride) + int(cache.max_seq_len) > n:
            raise ValueError(f"cache.rows holds {n} rows, B={B} sequences of stride "
                             f"{cache.seq_stride} need {(B - 1) * cache.seq_stride + cache.max_seq_len}")


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


@dataclass
class Geometry:
    heads: int
    d_nope: int = 128
    d_rope: int = D_ROPE
    d_latent: int = D_LATENT
    d_v: int = 128
    softmax_scale: float = 0.0  # <= 0: 1/sqrt(d_nope + d_rope)

    def c(self) -> Dims:
        return Dims(self.heads, self.d_nope, self.d_rope, self.d_latent, self.d_v,
                    float(self.softmax_scale))


@dataclass
class Cache:
    """Latent cache of one layer (see mla_cache_t).  rows: [n_rows, 576]
    (float32 / bfloat16 / uint8 e4m3 codes); row_scale: float32 [n_rows] for
    e4m3; seq_lens: int32 [B] on the device; block_table: int32 [B, max_pages]
    for the paged layout."""
    rows: torch.Tensor
    seq_lens: torch.Tensor
    max_seq_len: int
    row_scale: Optional[torch.Tensor] = None
    block_table: Optional[torch.Tensor] = None
    seq_stride: int = 0
    page_size: int = 0
    ring: bool = False  # contiguous rows used as rings of seq_stride slots

    def c(self) -> CacheDesc:
        mp = 0 if self.block_table is None else int(self.block_table.shape[1])
        return CacheDesc(dtype_code(self.rows), _ptr(self.rows), _ptr(self.row_scale),
                         int(self.page_size), int(self.seq_stride), _ptr(self.block_table), mp,
                         _ptr(self.seq_lens), int(self.max_seq_len), int(bool(self.ring)))


class Call:
    """One library call whose arguments were validated and marshalled once:
    calling it enqueues the same launch again (the buffers' contents may have
    changed since, not their addresses or shapes).  The ctypes structures the
    arguments point to are kept alive with it."""

    def __init__(self, name: str, args: tuple, keep: tuple):
        self.name = name
        self.fn = getattr(lib(), name)
        self.args = args
        self._keep = keep

    def __call__(self) -> None:
        _check(self.name, self.fn(*self.args))


def _launch(name: str, args: tuple, keep: tuple, prepare: bool):
    if prepare:
        return Call(name, args, keep)
    _check(name, getattr(lib(), name)(*args))
    return None


def _dims(geo: Geometry):
    return geo.heads, geo.d_latent + geo.d_rope


def mla_absorb_q_rope(geo: Geometry, q_nope: torch.Tensor, q_rope: torch.Tensor,
                      w_uk: torch.Tensor, positions: torch.Tensor, q_abs: torch.Tensor,
                      rope_base: float = 10000.0, stream=None, prepare: bool = False):
    """mla_absorb_q with q_R rotated by positions (int32 [B] on the device)."""
    B = int(q_nope.shape[0])
    H, W = _dims(geo)
    _need("q_nope", q_nope, (B, H, geo.d_nope), _FLOAT)
    _need("q_rope", q_rope, (B, H, geo.d_rope), _FLOAT)
    _need("w_uk", w_uk, (H, geo.d_nope, geo.d_latent), _FLOAT)
    _need("positions", positions, (B,), (torch.int32,))
    _need("q_abs", q_abs, (B, H, W), _FLOAT)
    _on_gpu(q_nope, q_rope, w_uk, positions, q_abs)
    d = geo.c()
    return _launch("mla_absorb_q_rope", (C.byref(d), B, _ptr(q_nope), _ptr(q_rope), dtype_code(q_nope),
                                 _ptr(w_uk), dtype_code(w_uk), _ptr(positions), float(rope_base),
                                 _ptr(q_abs), dtype_code(q_abs), _stream(stream),), (d,), prepare)


def mla_stream_probe(src: torch.Tensor, workgroups: int, tiles: int, paired: bool,
                     sink: torch.Tensor, stream=None, prepare: bool = False):
    """The decode's tile stream without its arithmetic (a measurement): src any
    contiguous device tensor (its bytes are streamed), sink int32 [workgroups]."""
    if not src.is_contiguous():
        raise ValueError("src must be contiguous")
    _need("sink", sink, (int(workgroups),), (torch.int32,))
    _on_gpu(src, sink)
    nbytes = src.numel() * src.element_size()
    return _launch("mla_stream_probe", (_ptr(src), nbytes, int(workgroups), int(tiles),
                                        1 if paired else 0, _ptr(sink), _stream(stream)), (),
                   prepare)


def mla_gqa_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   seq_lens: torch.Tensor, max_seq_len: int, o: torch.Tensor,
                   lse: Optional[torch.Tensor] = None, softmax_scale: float = 0.0,
                   stream=None, prepare: bool = False):
    """Grouped-query baseline decode: q [B, h, 128], k_cache / v_cache [B, h_kv,
    stride, 128] (bfloat16, h a multiple of h_kv; query head i reads key/value
    head i // (h / h_kv)), seq_lens int32 [B] on the device; o [B, h, 128]."""
    B, H, D = (int(x) for x in q.shape)
    if k_cache.dim() != 4:
        raise ValueError("k_cache must be [B, h_kv, stride, d_head]")
    Hkv, stride = int(k_cache.shape[1]), int(k_cache.shape[2])
    if Hkv < 1 or H % Hkv:
        raise ValueError(f"{Hkv} key/value heads do not divide {H} query heads")
    _need("q", q, (B, H, D), _FLOAT)
    _need("k_cache", k_cache, (B, Hkv, stride, D), (q.dtype,))
    _need("v_cache", v_cache, (B, Hkv, stride, D), (q.dtype,))
    _need("seq_lens", seq_lens, (B,), (torch.int32,))
    _need("o", o, (B, H, D), _FLOAT)
    _need("lse", lse, (B, H), (torch.float32,), optional=True)
    if not 0 <= int(max_seq_len) <= stride:
        raise ValueError("max_seq_len must lie in [0, stride]")
    _on_gpu(q, k_cache, v_cache, seq_lens, o, lse)
    return _launch("mla_gqa_decode", (B, H, Hkv, D, _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                      dtype_code(q), _ptr(seq_lens), stride, int(max_seq_len),
                                      float(softmax_scale), _ptr(o), dtype_code(o), _ptr(lse),
                                      _stream(stream)), (), prepare)


def mla_mha_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   seq_lens: torch.Tensor, max_seq_len: int, o: torch.Tensor,
                   lse: Optional[torch.Tensor] = None, softmax_scale: float = 0.0,
                   stream=None, prepare: bool = False):
    """MHA baseline decode: q [B, h, 128], k_cache / v_cache [B, h, stride, 128]
    (bfloat16), seq_lens int32 [B] on the device; o [B, h, 128]."""
    B, H, D = (int(x) for x in q.shape)
    if k_cache.dim() != 4 or int(k_cache.shape[1]) != H:
        raise ValueError("k_cache must be [B, h, stride, d_head]")
    stride = int(k_cache.shape[2])
    _need("q", q, (B, H, D), _FLOAT)
    _need("k_cache", k_cache, (B, H, stride, D), (q.dtype,))
    _need("v_cache", v_cache, (B, H, stride, D), (q.dtype,))
    _need("seq_lens", seq_lens, (B,), (torch.int32,))
    _need("o", o, (B, H, D), _FLOAT)
    _need("lse", lse, (B, H), (torch.float32,), optional=True)
    if not 0 <= int(max_seq_len) <= stride:
        raise ValueError("max_seq_len must lie in [0, stride]")
    _on_gpu(q, k_cache, v_cache, seq_lens, o, lse)
    return _launch("mla_mha_decode", (B, H, D, _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                      dtype_code(q), _ptr(seq_lens), stride, int(max_seq_len),
                                      float(softmax_scale), _ptr(o), dtype_code(o), _ptr(lse),
                                      _stream(stream)), (), prepare)


def mla_cache_append(geo: Geometry, c_kv: torch.Tensor, k_r: torch.Tensor,
                     positions: torch.Tensor, cache: Cache, stream=None, prepare: bool = False):
    """Write token positions[b] of every sequence b: c_kv [B, d_latent] and
    k_r [B, d_rope] (float32 or bfloat16) into cache.rows (and row_scale for
    an e4m3 cache).  positions: int32 [B] on the device."""
    B = int(c_kv.shape[0])
    _need("c_kv", c_kv, (B, geo.d_latent), _FLOAT)
    _need("k_r", k_r, (B, geo.d_rope), (c_kv.dtype,))
    _need("positions", positions, (B,), (torch.int32,))
    _need_cache(cache, B, geo)
    _on_gpu(c_kv, k_r, positions, *_cache_tensors(cache))
    d = geo.c()
    cd = cache.c()
    return _launch("mla_cache_append", (C.byref(d), B, _ptr(c_kv), _ptr(k_r), dtype_code(c_kv),
                                _ptr(positions), C.byref(cd), _stream(stream),), (d, cd), prepare)


def mla_cache_ring_grow(geo: Geometry, src: Cache, dst: Cache, stream=None,
                        prepare: bool = False):
    """Move every sequence's live window from the ring cache `src` into the
    ring cache `dst` (token t to row t % dst.seq_stride); lengths from src."""
    B = int(src.seq_lens.shape[0])
    for name, c in (("src", src), ("dst", dst)):
        if not c.ring:
            raise ValueError(f"{name} must be a ring cache")
        _need_cache(c, B, geo) if c is src else _need_cache(
            Cache(rows=c.rows, seq_lens=src.seq_lens, max_seq_len=0, row_scale=c.row_scale,
                  seq_stride=c.seq_stride, ring=True), B, geo)
    if src.rows.dtype != dst.rows.dtype:
        raise TypeError("src and dst rings must have the same dtype")
    _on_gpu(*_cache_tensors(src), *_cache_tensors(dst))
    cs, cd = src.c(), dst.c()
    return _launch("mla_cache_ring_grow", (B, C.byref(cs), C.byref(cd), _stream(stream)),
                   (cs, cd), prepare)


def mla_absorb_q(geo: Geometry, q_nope: torch.Tensor, q_rope: torch.Tensor, w_uk: torch.Tensor,
                 q_abs: torch.Tensor, q_abs_scale: Optional[torch.Tensor] = None,
                 stream=None, prepare: bool = False):
    """q_nope [B, h, d_nope], q_rope [B, h, d_rope], w_uk [h, d_nope, 512] ->
    q_abs [B, h, 576] (float32, bfloat16, or e4m3 codes as uint8 /
    float8_e4m3fn with q_abs_scale float32 [B, h])."""
    B = int(q_nope.shape[0])
    H, W = _dims(geo)
    _need("q_nope", q_nope, (B, H, geo.d_nope), _FLOAT)
    _need("q_rope", q_rope, (B, H, geo.d_rope), _FLOAT)
    _need("w_uk", w_uk, (H, geo.d_nope, geo.d_latent), _FLOAT)
    _need("q_abs", q_abs, (B, H, W), _CACHE_DT)
    _need("q_abs_scale", q_abs_scale, (B, H), (torch.float32,), optional=True)
    _on_gpu(q_nope, q_rope, w_uk, q_abs, q_abs_scale)
    d = geo.c()
    return _launch("mla_absorb_q", (C.byref(d), B, _ptr(q_nope), _ptr(q_rope), dtype_code(q_nope),
                            _ptr(w_uk), dtype_code(w_uk), _ptr(q_abs), dtype_code(q_abs),
                            _ptr(q_abs_scale), _stream(stream),), (d,), prepare)


def _need_parts(geo: Geometry, lead: tuple, S: int, u_part, lse_part) -> None:
    H = geo.heads
    _need("u_part", u_part, (*lead, S, H, geo.d_latent), _FLOAT)
    _need("lse_part", lse_part, (*lead, S, H), (torch.float32,))


def mla_decode(geo: Geometry, q_abs: torch.Tensor, cache: Cache, num_splits: int,
               u_part: torch.Tensor, lse_part: torch.Tensor,
               q_abs_scale: Optional[torch.Tensor] = None, stream=None, prepare: bool = False):
    """q_abs [B, h, 576]; u_part [B, S, h, 512]; lse_part [B, S, h]."""
    B = int(q_abs.shape[0])
    H, W = _dims(geo)
    _need("q_abs", q_abs, (B, H, W), _CACHE_DT)
    _need("q_abs_scale", q_abs_scale, (B, H), (torch.float32,), optional=True)
    _need_parts(geo, (B,), int(num_splits), u_part, lse_part)
    _need_cache(cache, B, geo)
    _on_gpu(q_abs, q_abs_scale, u_part, lse_part, *_cache_tensors(cache))
    d = geo.c()
    cd = cache.c()
    return _launch("mla_decode", (C.byref(d), B, _ptr(q_abs), dtype_code(q_abs), _ptr(q_abs_scale),
                          C.byref(cd), int(num_splits), _ptr(u_part), dtype_code(u_part),
                          _ptr(lse_part), _stream(stream),), (d, cd), prepare)


def mla_decode_multi(geo: Geometry, q_abs: torch.Tensor, cache: Cache, num_splits: int,
                     u_part: torch.Tensor, lse_part: torch.Tensor, stream=None, prepare: bool = False):
    """Multi-token decode: q_abs [B, q_len, h, 576]; u_part [B, q_len, S, h,
    512]; lse_part [B, q_len, S, h] (the last q_len cached rows are the new
    tokens, attended causally)."""
    if q_abs.dim() != 4:
        raise ValueError("q_abs must be [B, q_len, h, 576]")
    B, QL = int(q_abs.shape[0]), int(q_abs.shape[1])
    H, W = _dims(geo)
    _need("q_abs", q_abs, (B, QL, H, W), _FLOAT)
    _need_parts(geo, (B, QL), int(num_splits), u_part, lse_part)
    _need_cache(cache, B, geo)
    _on_gpu(q_abs, u_part, lse_part, *_cache_tensors(cache))
    d = geo.c()
    cd = cache.c()
    return _launch("mla_decode_multi", (C.byref(d), B, QL, _ptr(q_abs), dtype_code(q_abs), C.byref(cd),
                                int(num_splits), _ptr(u_part), dtype_code(u_part), _ptr(lse_part),
                                _stream(stream),), (d, cd), prepare)


KERNEL_AUTO, KERNEL_H64, KERNEL_H64_BALANCED = 0, 1, 4  # mla_decode_kernel_t (2, 3: retired)


def mla_decode_ex(geo: Geometry, q_abs: torch.Tensor, cache: Cache, num_splits: int,
                  u_part: torch.Tensor, lse_part: torch.Tensor, kernel: int = KERNEL_AUTO,
                  stream=None, prepare: bool = False):
    """mla_decode (q_abs [B, h, 576]) or mla_decode_multi (q_abs [B, q_len, h,
    576]) with the decode kernel chosen by the caller (KERNEL_*)."""
    B = int(q_abs.shape[0])
    QL = int(q_abs.shape[1]) if q_abs.dim() == 4 else 1
    H, W = _dims(geo)
    lead = (B, QL) if q_abs.dim() == 4 else (B,)
    _need("q_abs", q_abs, (*lead, H, W), _FLOAT)
    _need_parts(geo, lead, int(num_splits), u_part, lse_part)
    _need_cache(cache, B, geo)
    _on_gpu(q_abs, u_part, lse_part, *_cache_tensors(cache))
    d = geo.c()
    cd = cache.c()
    return _launch("mla_decode_ex", (C.byref(d), B, QL, _ptr(q_abs), dtype_code(q_abs), C.byref(cd),
                             int(num_splits), _ptr(u_part), dtype_code(u_part), _ptr(lse_part),
                             int(kernel), _stream(stream),), (d, cd), prepare)


def mla_combine(geo: Geometry, u_part: torch.Tensor, lse_part: torch.Tensor, u: torch.Tensor,
                lse: Optional[torch.Tensor] = None, stream=None, prepare: bool = False):
    """u_part [B, S, h, 512], lse_part [B, S, h] -> u [B, h, 512], lse [B, h]."""
    B, S = int(u_part.shape[0]), int(u_part.shape[1])
    H = geo.heads
    _need_parts(geo, (B,), S, u_part, lse_part)
    _need("u", u, (B, H, geo.d_latent), _FLOAT)
    _need("lse", lse, (B, H), (torch.float32,), optional=True)
    _on_gpu(u_part, lse_part, u, lse)
    d = geo.c()
    return _launch("mla_combine", (C.byref(d), B, S, _ptr(u_part), dtype_code(u_part), _ptr(lse_part),
                           _ptr(u), dtype_code(u), _ptr(lse), _stream(stream),), (d,), prepare)


def mla_up_proj(geo: Geometry, u: torch.Tensor, w_uv: torch.Tensor, o: torch.Tensor,
                stream=None, prepare: bool = False):
    """u [B, h, 512], w_uv [h, d_v, 512] -> o [B, h, d_v]."""
    B = int(u.shape[0])
    H = geo.heads
    _need("u", u, (B, H, geo.d_latent), _FLOAT)
    _need("w_uv", w_uv, (H, geo.d_v, geo.d_latent), _FLOAT)
    _need("o", o, (B, H, geo.d_v), _FLOAT)
    _on_gpu(u, w_uv, o)
    d = geo.c()
    return _launch("mla_up_proj", (C.byref(d), B, _ptr(u), dtype_code(u), _ptr(w_uv), dtype_code(w_uv),
                           _ptr(o), dtype_code(o), _stream(stream),), (d,), prepare)


def mla_combine_up_proj(geo: Geometry, u_part: torch.Tensor, lse_part: torch.Tensor,
                        w_uv: torch.Tensor, o: torch.Tensor, u: Optional[torch.Tensor] = None,
                        lse: Optional[torch.Tensor] = None, stream=None, prepare: bool = False):
    """u_part [B, S, h, 512], lse_part [B, S, h], w_uv [h, d_v, 512] ->
    o [B, h, d_v]; optionally u [B, h, 512] (bfloat16) and lse [B, h]."""
    B, S = int(u_part.shape[0]), int(u_part.shape[1])
    H = geo.heads
    if u is not None and u.dtype != torch.bfloat16:
        raise TypeError("mla_combine_up_proj stores u as bfloat16 only")
    _need_parts(geo, (B,), S, u_part, lse_part)
    _need("w_uv", w_uv, (H, geo.d_v, geo.d_latent), _FLOAT)
    _need("o", o, (B, H, geo.d_v), _FLOAT)
    _need("u", u, (B, H, geo.d_latent), (torch.bfloat16,), optional=True)
    _need("lse", lse, (B, H), (torch.float32,), optional=True)
    _on_gpu(u_part, lse_part, w_uv, o, u, lse)
    d = geo.c()
    return _launch("mla_combine_up_proj", (C.byref(d), B, S, _ptr(u_part), dtype_code(u_part),
                                   _ptr(lse_part), _ptr(w_uv), dtype_code(w_uv), _ptr(o),
                                   dtype_code(o), _ptr(u), _ptr(lse), _stream(stream),), (d,), prepare)


def mla_decode_combine_up_proj_noalloc(geo: Geometry, q_abs: torch.Tensor, cache: Cache,
                                       num_splits: int, w_uv: torch.Tensor, o: torch.Tensor,
                                       u: Optional[torch.Tensor] = None,
                                       lse: Optional[torch.Tensor] = None, stream=None,
                                       prepare: bool = False):
    """mla_decode + mla_combine_up_proj with the split partials in the
    library's static device scratch (no allocation by anyone): q_abs [B, h,
    576], w_uv [h, d_v, 512] -> o [B, h, d_v]; optionally u [B, h, 512]
    (bfloat16) and lse [B, h].  B * num_splits * h <= 65536."""
    B = int(q_abs.shape[0])
    H, W = _dims(geo)
    if u is not None and u.dtype != torch.bfloat16:
        raise TypeError("the merged u is stored as bfloat16 only")
    _need("q_abs", q_abs, (B, H, W), _FLOAT)
    _need("w_uv", w_uv, (H, geo.d_v, geo.d_latent), _FLOAT)
    _need("o", o, (B, H, geo.d_v), _FLOAT)
    _need("u", u, (B, H, geo.d_latent), (torch.bfloat16,), optional=True)
    _need("lse", lse, (B, H), (torch.float32,), optional=True)
    _need_cache(cache, B, geo)
    _on_gpu(q_abs, w_uv, o, u, lse, *_cache_tensors(cache))
    d = geo.c()
    cd = cache.c()
    return _launch("mla_decode_combine_up_proj_noalloc",
                   (C.byref(d), B, _ptr(q_abs), dtype_code(q_abs), C.byref(cd), int(num_splits),
                    _ptr(w_uv), dtype_code(w_uv), _ptr(o), dtype_code(o), _ptr(u), _ptr(lse),
                    _stream(stream)), (d, cd), prepare)


def mla_prefill_rebuild_kv(geo: Geometry, cache: Cache, w_uk: torch.Tensor, w_uv: torch.Tensor,
                           k: torch.Tensor, vt: torch.Tensor,
                           rebuild_from: Optional[torch.Tensor] = None, stream=None,
                           prepare: bool = False):
    """Naive-form keys k [B, h, kv_stride, 192] and transposed values vt [B, h,
    128, kv_stride] (bfloat16) of the cached tokens [rebuild_from[b], L_b)."""
    B = int(cache.seq_lens.shape[0])
    H = geo.heads
    if k.dim() != 4:
        raise ValueError("k must be [B, h, kv_stride, d_nope + d_rope]")
    S = int(k.shape[2])
    _need("k", k, (B, H, S, geo.d_nope + geo.d_rope), (torch.bfloat16,))
    _need("vt", vt, (B, H, geo.d_v, S), (torch.bfloat16,))
    _need("w_uk", w_uk, (H, geo.d_nope, geo.d_latent), (torch.bfloat16,))
    _need("w_uv", w_uv, (H, geo.d_v, geo.d_latent), (torch.bfloat16,))
    _need("rebuild_from", rebuild_from, (B,), (torch.int32,), optional=True)
    _need_cache(cache, B, geo)
    _on_gpu(k, vt, w_uk, w_uv, rebuild_from, *_cache_tensors(cache))
    d = geo.c()
    cd = cache.c()
    return _launch("mla_prefill_rebuild_kv",
                   (C.byref(d), B, C.byref(cd), _ptr(rebuild_from), _ptr(w_uk), _ptr(w_uv),
                    dtype_code(w_uk), _ptr(k), _ptr(vt), S, _stream(stream)), (d, cd), prepare)


def mla_prefill_attn(geo: Geometry, q: torch.Tensor, q_lens: torch.Tensor, k: torch.Tensor,
                     vt: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int, o: torch.Tensor,
                     lse: Optional[torch.Tensor] = None, stream=None, prepare: bool = False):
    """Causal attention of each sequence's last q_lens[b] cached tokens (queries
    q [B, q_len, h, 192] = [q_C | q_R], bfloat16) over k / vt from
    mla_prefill_rebuild_kv -> o [B, q_len, h, 128], lse [B, q_len, h]."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, q_len, h, 192] and k [B, h, kv_stride, 192]")
    B, QL = int(q.shape[0]), int(q.shape[1])
    H = geo.heads
    S = int(k.shape[2])
    W = geo.d_nope + geo.d_rope
    _need("q", q, (B, QL, H, W), (torch.bfloat16,))
    _need("q_lens", q_lens, (B,), (torch.int32,))
    _need("k", k, (B, H, S, W), (torch.bfloat16,))
    _need("vt", vt, (B, H, geo.d_v, S), (torch.bfloat16,))
    _need("seq_lens", seq_lens, (B,), (torch.int32,))
    _need("o", o, (B, QL, H, geo.d_v), _FLOAT)
    _need("lse", lse, (B, QL, H), (torch.float32,), optional=True)
    if not 0 <= int(max_seq_len) <= S:
        raise ValueError("max_seq_len must lie in [0, kv_stride]")
    _on_gpu(q, q_lens, k, vt, seq_lens, o, lse)
    d = geo.c()
    return _launch("mla_prefill_attn",
                   (C.byref(d), B, QL, _ptr(q_lens), _ptr(q), dtype_code(q), _ptr(k), _ptr(vt), S,
                    _ptr(seq_lens), int(max_seq_len), _ptr(o), dtype_code(o), _ptr(lse),
                    _stream(stream)), (d,), prepare)


def split_chunk(max_seq_len: int, num_splits: int) -> int:
    """Tokens per split range (mirrors the rule stated in include/mla.h)."""
    if max_seq_len <= 0:
        return 0
    per = TILE_TOKENS * num_splits
    return -(-max_seq_len // per) * TILE_TOKENS


class DecodeStep:
    """One MLA decode step of one layer: the four library calls in order, with
    the intermediate buffers allocated once (torch allocator) and reused.

    q_nope [B, h, d_nope], q_rope [B, h, d_rope], w_uk [h, d_nope, 512],
    w_uv [h, d_v, 512] (float32 or bfloat16); the cache as `Cache`.
    act_dtype is the dtype of q_abs / u; part_dtype of the split partials.
    fp8_query: q_abs in E4M3 with one factor per (sequence, head) (an fp8
    cache only; the decode then runs on the fp8 matrix cores)."""

    def __init__(self, geo: Geometry, batch: int, num_splits: int, device="cuda",
                 act_dtype=torch.bfloat16, part_dtype=torch.bfloat16, out_dtype=torch.bfloat16,
                 kernel: int = KERNEL_AUTO, fp8_query: bool = False):
        self.geo = geo
        self.kernel = int(kernel)
        self.B = batch
        self.S = int(num_splits)
        h = geo.heads
        w = geo.d_latent + geo.d_rope
        if fp8_query and self.kernel != KERNEL_AUTO:
            raise ValueError("an fp8 query runs its own kernel (KERNEL_AUTO)")
        self.q_abs = torch.empty(batch, h, w, dtype=torch.uint8 if fp8_query else act_dtype,
                                 device=device)
        self.q_abs_scale = (torch.empty(batch, h, dtype=torch.float32, device=device)
                            if fp8_query else None)
        self.u_part = torch.empty(batch, self.S, h, geo.d_latent, dtype=part_dtype, device=device)
        self.lse_part = torch.empty(batch, self.S, h, dtype=torch.float32, device=device)
        self.u = (self.u_part.view(batch, h, geo.d_latent) if self.S == 1
                  else torch.empty(batch, h, geo.d_latent, dtype=part_dtype, device=device))
        self.lse = (self.lse_part.view(batch, h) if self.S == 1
                    else torch.empty(batch, h, dtype=torch.float32, device=device))
        self.o = torch.empty(batch, h, geo.d_v, dtype=out_dtype, device=device)

    def fused_tail(self, w_uv: torch.Tensor) -> bool:
        """Whether run() merges the splits and applies W_UV in one launch
        (mla_combine_up_proj): several splits, bf16 W_UV and u."""
        return (self.S > 1 and w_uv.dtype == torch.bfloat16 and self.u.dtype == torch.bfloat16
                and self.geo.d_v % 16 == 0)

    def run(self, q_nope, q_rope, w_uk, w_uv, cache: Cache, stream=None,
            fused: bool = True) -> torch.Tensor:
        mla_absorb_q(self.geo, q_nope, q_rope, w_uk, self.q_abs, self.q_abs_scale, stream=stream)
        if self.kernel == KERNEL_AUTO:
            mla_decode(self.geo, self.q_abs, cache, self.S, self.u_part, self.lse_part,
                       q_abs_scale=self.q_abs_scale, stream=stream)
        else:
            mla_decode_ex(self.geo, self.q_abs, cache, self.S, self.u_part, self.lse_part,
                          kernel=self.kernel, stream=stream)
        if fused and self.fused_tail(w_uv):
            mla_combine_up_proj(self.geo, self.u_part, self.lse_part, w_uv, self.o, self.u,
                                self.lse, stream=stream)
            return self.o
        if self.S > 1:
            mla_combine(self.geo, self.u_part, self.lse_part, self.u, self.lse, stream=stream)
        mla_up_proj(self.geo, self.u, w_uv, self.o, stream=stream)
        return self.o

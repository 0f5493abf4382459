"""Shared helpers of the GPU tests: upload seeded synthetic inputs, run one
decode step through the library's C ABI, and compare with the CPU oracle on
chosen (sequence, head) pairs."""

from __future__ import annotations

import numpy as np
import torch

import mla_latent_kv_15_amd as mla
import oracle
from tests.device_inputs import TORCH_DT, DeviceInputs, act_torch_dtype, bits_to_tensor  # noqa: F401

# max|gpu - oracle| <= TOL * max|oracle| per compared quantity
TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 6e-2}


def run_step(dev: DeviceInputs, num_splits: int, part_dtype=None, out_dtype=None,
             kernel: int = mla.KERNEL_AUTO, fp8_query: bool = False):
    """absorb -> decode -> combine -> up_proj.  Returns the DecodeStep (its
    buffers hold q_abs, u_part, lse_part, u, lse, o)."""
    wl = dev.wl
    act = act_torch_dtype(wl)
    step = mla.DecodeStep(dev.geo, wl.batch, num_splits, act_dtype=act,
                          part_dtype=part_dtype or act,
                          out_dtype=out_dtype or TORCH_DT[wl.out_dtype], kernel=kernel,
                          fp8_query=fp8_query)
    step.run(dev.q_nope, dev.q_rope, dev.w_uk, dev.w_uv, dev.cache)
    torch.cuda.synchronize()
    return step


def sample_pairs(B: int, H: int, n_b: int = 4, n_h: int = 4, seq_lens=None):
    """A deterministic spread of (b, h) pairs: first/last sequences and heads
    plus interior ones; sequences of length 0 are kept (they must give 0)."""
    bs = sorted(set(np.linspace(0, B - 1, n_b).round().astype(int).tolist()))
    hs = sorted(set(np.linspace(0, H - 1, n_h).round().astype(int).tolist()))
    return [(b, h) for b in bs for h in hs]


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), "non-finite GPU output"
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    diff = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    if scale == 0.0:
        return diff
    return diff / scale


def check_against_oracle(dev: DeviceInputs, step: mla.DecodeStep, pairs, tol: float):
    """o, u and lse of the selected pairs against the oracle.  Returns the
    three relative errors."""
    o_ref, lse_ref, u_ref = oracle.decode_inputs(dev.inp, sel=pairs, want_u=True)
    o = step.o.float().cpu().numpy()
    u = step.u.float().cpu().numpy()
    lse = step.lse.float().cpu().numpy()
    o_got = np.stack([o[b, h] for b, h in pairs])
    u_got = np.stack([u[b, h] for b, h in pairs])
    lse_got = np.array([lse[b, h] for b, h in pairs])
    e_o = rel_err(o_got, o_ref)
    e_u = rel_err(u_got, u_ref)
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse_got), fin), "empty-sequence lse must be -inf"
    assert np.all(lse_got[~fin] == -np.inf)
    e_l = float(np.max(np.abs(lse_got[fin] - lse_ref[fin]))) if fin.any() else 0.0
    assert e_o <= tol, f"o: max err {e_o:.3e} > {tol:g} of max|o|"
    assert e_u <= tol, f"u: max err {e_u:.3e} > {tol:g} of max|u|"
    # lse is a log: an absolute error of tol is a relative error of tol in exp(lse)
    assert e_l <= tol, f"lse: max abs err {e_l:.3e} > {tol:g}"
    return e_o, e_u, e_l


ROW_START_WEIGHT = 5


def balanced_pieces(att, S: int, HG: int, workgroups: int = 256):
    """The balanced partition of mla_decode_ex(MLA_KERNEL_H64_BALANCED), as the
    C header states it: rows v laid end to end, a row attending att[v] > 0
    tokens weighing 5 + n_v (n_v = ceil(att[v]/32) tiles, after its 5 units of
    start weight), an empty row 0; the total weight N cut into G spans
    [w N / G, (w+1) N / G) with G = min(workgroups / HG, max(1, N // ceil(n_max /
    (S-1)))) (1 if N = 0), n_max the largest row weight.  Returns {(v, split):
    (t_begin, t_end) or None (empty)} for every row and split."""
    att = [int(a) for a in att]
    n = [(a + 31) // 32 for a in att]
    wt = [ROW_START_WEIGHT + x if x else 0 for x in n]
    N, nmax = sum(wt), max(wt) if wt else 0
    G = 1 if N == 0 else min(max(1, workgroups // HG), max(1, N // -(-nmax // (S - 1))))
    span_of = lambda x: min(G - 1, ((x + 1) * G - 1) // N) if N else 0  # the span holding unit x
    out = {}
    pre = 0
    for v, (a, nv) in enumerate(zip(att, n)):
        if nv == 0:
            for p in range(S):
                out[(v, p)] = None
            continue
        f0 = pre + ROW_START_WEIGHT  # the row's first tile
        w0, w1 = span_of(f0), span_of(f0 + nv - 1)
        assert w1 - w0 < S
        for w in range(w0, w1 + 1):
            lo, hi = w * N // G, (w + 1) * N // G
            t0 = 32 * (max(lo, f0) - f0)
            t1 = min(32 * (min(hi, f0 + nv) - f0), a)
            out[(v, w - w0)] = (t0, t1)
        for p in range(w1 - w0 + 1, S):
            out[(v, p)] = None
        pre += wt[v]
    return out


def ranges_per_split(B: int, q_len: int, S: int, heads: int, grouped: bool) -> int:
    """R of mla_decode's merged range groups, as the C header states it: with
    an FP8 query, or a BF16 cache and S >= 32 (grouped), R = min(S, max(1,
    floor(B q_len S ceil(h/64) / 256))); else 1.  Split g then covers ranges
    gR .. gR+R-1 and the splits from ceil(S / R) on are empty."""
    if not grouped:
        return 1
    return min(S, max(1, (B * q_len * S * -(-heads // 64)) // 256))

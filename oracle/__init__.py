"""CPU oracle for MLA decode — TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package.  It wraps liboracle.so (oracle.c: plain float64 C) with
numpy marshalling and shares nothing with the GPU library.
"""

from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

import numpy as np

from .build import LIB, build

F32, BF16, E4M3, F64 = 0, 1, 2, 3
_DT = {"f32": F32, "bf16": BF16, "fp8": E4M3, "e4m3": E4M3, "f64": F64}
_NP = {F32: np.float32, BF16: np.uint16, E4M3: np.uint8, F64: np.float64}

_lib = None


class _Problem(C.Structure):
    _fields_ = [
        ("B", C.c_int32), ("H", C.c_int32), ("d_nope", C.c_int32), ("d_rope", C.c_int32),
        ("d_latent", C.c_int32), ("d_v", C.c_int32), ("scale", C.c_double),
        ("q_nope", C.c_void_p), ("q_rope", C.c_void_p), ("q_dtype", C.c_int32),
        ("w_uk", C.c_void_p), ("w_uv", C.c_void_p), ("w_dtype", C.c_int32),
        ("rows", C.c_void_p), ("row_scale", C.c_void_p), ("cache_dtype", C.c_int32),
        ("page_size", C.c_int32), ("seq_stride", C.c_int64), ("block_table", C.c_void_p),
        ("max_pages", C.c_int32), ("seq_lens", C.c_void_p), ("ring", C.c_int32),
    ]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = C.CDLL(LIB)
        L.oracle_mla_decode.restype = C.c_int
        L.oracle_mla_decode.argtypes = [C.POINTER(_Problem), C.c_void_p, C.c_void_p, C.c_int32,
                                        C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                        C.c_void_p]
        L.oracle_rebuild_kv.restype = C.c_int
        L.oracle_rebuild_kv.argtypes = [C.POINTER(_Problem), C.c_int32, C.c_int32, C.c_int32,
                                        C.c_void_p, C.c_void_p]
        L.oracle_absorbed_decode.restype = C.c_int
        L.oracle_absorbed_decode.argtypes = [C.POINTER(_Problem), C.c_void_p, C.c_int32,
                                             C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32,
                                             C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                             C.c_void_p]
        L.oracle_quantize_e4m3_rows.restype = C.c_int
        L.oracle_quantize_e4m3_rows.argtypes = [C.c_int64, C.c_int32, C.c_void_p, C.c_void_p,
                                                C.c_void_p]
        L.oracle_absorb_q.restype = C.c_int
        L.oracle_absorb_q.argtypes = [C.c_int32] * 5 + [C.c_void_p, C.c_void_p, C.c_int32,
                                                        C.c_void_p, C.c_int32, C.c_void_p]
        L.oracle_combine.restype = C.c_int
        L.oracle_combine.argtypes = [C.c_int32] * 4 + [C.c_void_p] * 4
        L.oracle_up_proj.restype = C.c_int
        L.oracle_up_proj.argtypes = [C.c_int32] * 4 + [C.c_void_p, C.c_void_p, C.c_int32,
                                                       C.c_void_p]
        L.oracle_decode_bf16.restype = C.c_double
        L.oracle_decode_bf16.argtypes = [C.c_uint16]
        L.oracle_decode_e4m3.restype = C.c_double
        L.oracle_decode_e4m3.argtypes = [C.c_uint8]
        L.oracle_decode_array.restype = None
        L.oracle_decode_array.argtypes = [C.c_void_p, C.c_int32, C.c_int64, C.c_void_p]
        L.oracle_mla_cache_bytes_per_token.restype = C.c_int64
        L.oracle_mla_cache_bytes_per_token.argtypes = [C.c_int32] * 4
        L.oracle_mha_cache_bytes.restype = C.c_int64
        L.oracle_mha_cache_bytes.argtypes = [C.c_int64] * 5
        L.oracle_cache_append.restype = C.c_int
        L.oracle_cache_append.argtypes = [C.c_int32] * 3 + [C.c_void_p, C.c_void_p, C.c_int32,
                                                            C.c_void_p, C.c_void_p, C.c_int32,
                                                            C.c_void_p, C.c_int32, C.c_int64,
                                                            C.c_void_p, C.c_int32, C.c_int32]
        L.oracle_ring_grow.restype = C.c_int
        L.oracle_ring_grow.argtypes = [C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p,
                                       C.c_int64, C.c_void_p, C.c_void_p, C.c_int64]
        L.oracle_mha_decode.restype = C.c_int
        L.oracle_mha_decode.argtypes = [C.c_int32] * 4 + [C.c_void_p] * 3 + [
            C.c_int32, C.c_void_p, C.c_int64, C.c_double, C.c_void_p, C.c_void_p]
        L.oracle_gqa_decode.restype = C.c_int
        L.oracle_gqa_decode.argtypes = [C.c_int32] * 5 + [C.c_void_p] * 3 + [
            C.c_int32, C.c_void_p, C.c_int64, C.c_double, C.c_void_p, C.c_void_p]
        L.oracle_rope.restype = C.c_int
        L.oracle_rope.argtypes = [C.c_int32] * 3 + [C.c_void_p, C.c_int32, C.c_void_p,
                                                    C.c_double, C.c_void_p]
        L.oracle_rope_inv_freq.restype = None
        L.oracle_rope_inv_freq.argtypes = [C.c_int32, C.c_double, C.c_void_p]
        L.oracle_encode_e4m3.restype = C.c_uint8
        L.oracle_encode_e4m3.argtypes = [C.c_float]
        L.oracle_num_threads.restype = C.c_int
        L.oracle_num_threads.argtypes = []
        _lib = L
    return _lib


def _dt(x) -> int:
    return _DT[x] if isinstance(x, str) else int(x)


def _arr(a, dtype_code) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=_NP[dtype_code])


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def decode(q_nope, q_rope, q_dtype, w_uk, w_uv, w_dtype, rows, cache_dtype, seq_lens, *,
           row_scale=None, page_size: int = 0, seq_stride: Optional[int] = None,
           block_table=None, scale: Optional[float] = None,
           sel: Optional[Sequence[tuple]] = None, t_begin=None, t_end=None,
           want_u: bool = False, ring: bool = False):
    """Naive MLA decode.  Arrays hold stored bits (float32 / uint16 bf16 /
    uint8 e4m3 / float64).  Returns (o [n, d_v], lse [n], u [n, d_latent] or
    None) as float64, for the selected (b, h) pairs or all B*H in order."""
    qd, wd, cd = _dt(q_dtype), _dt(w_dtype), _dt(cache_dtype)
    q_nope = _arr(q_nope, qd)
    q_rope = _arr(q_rope, qd)
    w_uk = _arr(w_uk, wd)
    w_uv = _arr(w_uv, wd)
    rows = _arr(rows, cd)
    B, H, dn = q_nope.shape
    dr = q_rope.shape[2]
    dl = w_uk.shape[2]
    dv = w_uv.shape[1]
    assert rows.shape[-1] == dl + dr
    seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    rs = None if row_scale is None else np.ascontiguousarray(row_scale, dtype=np.float32)
    bt = None if block_table is None else np.ascontiguousarray(block_table, dtype=np.int32)
    if seq_stride is None:
        seq_stride = int(seq_lens.max()) if B else 0
    P = _Problem(B, H, dn, dr, dl, dv, float(scale) if scale else 0.0,
                 _ptr(q_nope), _ptr(q_rope), qd, _ptr(w_uk), _ptr(w_uv), wd,
                 _ptr(rows), _ptr(rs), cd, int(page_size), int(seq_stride), _ptr(bt),
                 0 if bt is None else int(bt.shape[1]), _ptr(seq_lens), int(bool(ring)))
    if sel is None:
        n = B * H
        sb = sh = None
    else:
        sel = list(sel)
        n = len(sel)
        sb = np.ascontiguousarray([s[0] for s in sel], dtype=np.int32)
        sh = np.ascontiguousarray([s[1] for s in sel], dtype=np.int32)
    tb = None if t_begin is None else np.ascontiguousarray(t_begin, dtype=np.int32)
    te = None if t_end is None else np.ascontiguousarray(t_end, dtype=np.int32)
    o = np.zeros((n, dv), dtype=np.float64)
    lse = np.zeros(n, dtype=np.float64)
    u = np.zeros((n, dl), dtype=np.float64) if want_u else None
    rc = lib().oracle_mla_decode(C.byref(P), _ptr(sb), _ptr(sh), n, _ptr(tb), _ptr(te),
                                 _ptr(o), _ptr(lse), _ptr(u))
    if rc != 0:
        raise ValueError(f"oracle_mla_decode failed: {rc}")
    return o, lse, u


def rebuild_kv(q_nope, q_rope, q_dtype, w_uk, w_uv, w_dtype, rows, cache_dtype, seq_lens, b,
               t_begin, t_end, *, row_scale=None, page_size: int = 0,
               seq_stride: Optional[int] = None, block_table=None):
    """The naive form's keys and values of sequence b, tokens [t_begin, t_end):
    (k [H, n, d_nope + d_rope], v [H, n, d_v]) float64 (arguments as decode)."""
    qd, wd, cd = _dt(q_dtype), _dt(w_dtype), _dt(cache_dtype)
    q_nope, q_rope = _arr(q_nope, qd), _arr(q_rope, qd)
    w_uk, w_uv, rows = _arr(w_uk, wd), _arr(w_uv, wd), _arr(rows, cd)
    B, H, dn = q_nope.shape
    dr, dl, dv = q_rope.shape[2], w_uk.shape[2], w_uv.shape[1]
    seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    rs = None if row_scale is None else np.ascontiguousarray(row_scale, dtype=np.float32)
    bt = None if block_table is None else np.ascontiguousarray(block_table, dtype=np.int32)
    if seq_stride is None:
        seq_stride = int(seq_lens.max()) if B else 0
    P = _Problem(B, H, dn, dr, dl, dv, 0.0, _ptr(q_nope), _ptr(q_rope), qd, _ptr(w_uk),
                 _ptr(w_uv), wd, _ptr(rows), _ptr(rs), cd, int(page_size), int(seq_stride),
                 _ptr(bt), 0 if bt is None else int(bt.shape[1]), _ptr(seq_lens), 0)
    n = int(t_end) - int(t_begin)
    k = np.zeros((H, n, dn + dr), dtype=np.float64)
    v = np.zeros((H, n, dv), dtype=np.float64)
    rc = lib().oracle_rebuild_kv(C.byref(P), int(b), int(t_begin), int(t_end), _ptr(k), _ptr(v))
    if rc != 0:
        raise ValueError(f"oracle_rebuild_kv failed: {rc}")
    return k, v


def rebuild_kv_inputs(inp, b, t_begin, t_end):
    """rebuild_kv() on a synth.MLAInputs-like object."""
    wl = inp.wl
    return rebuild_kv(inp.q_nope, inp.q_rope, wl.act_dtype, inp.w_uk, inp.w_uv, wl.act_dtype,
                      inp.rows, wl.cache_dtype, inp.seq_lens, b, t_begin, t_end,
                      row_scale=inp.row_scale, page_size=wl.page_size,
                      seq_stride=inp.seq_stride, block_table=inp.block_table)


def decode_inputs(inp, sel=None, want_u=False, t_begin=None, t_end=None, scale=None,
                  ring=False):
    """decode() on a synth.MLAInputs-like object (duck-typed)."""
    wl = inp.wl
    return decode(inp.q_nope, inp.q_rope, wl.act_dtype, inp.w_uk, inp.w_uv, wl.act_dtype,
                  inp.rows, wl.cache_dtype, inp.seq_lens, row_scale=inp.row_scale,
                  page_size=wl.page_size, seq_stride=inp.seq_stride,
                  block_table=inp.block_table, scale=scale, sel=sel, t_begin=t_begin,
                  t_end=t_end, want_u=want_u, ring=ring)


def absorbed_decode(q_abs, q_dtype, rows, cache_dtype, seq_lens, *, q_scale=None,
                    row_scale=None, page_size: int = 0, seq_stride: Optional[int] = None,
                    block_table=None, scale: Optional[float] = None, d_nope: int = 128,
                    w_uv=None, w_dtype="bf16", sel: Optional[Sequence[tuple]] = None,
                    t_begin=None, t_end=None, ring: bool = False):
    """Absorbed-form attention for a given q_abs [B, H, d_latent + d_rope]
    (stored bits in q_dtype; E4M3 with q_scale [B, H]).  Returns (u [n,
    d_latent], lse [n], o [n, d_v] or None) float64 for the selected (b, h)
    pairs or all B*H in order; o needs w_uv [H, d_v, d_latent]."""
    qd, cd, wd = _dt(q_dtype), _dt(cache_dtype), _dt(w_dtype)
    q_abs = _arr(q_abs, qd)
    rows = _arr(rows, cd)
    B, H, w = q_abs.shape
    dr = 64 if w > 64 else 0
    dl = w - dr
    assert rows.shape[-1] == w
    seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    qs = None if q_scale is None else np.ascontiguousarray(q_scale, dtype=np.float32)
    rs = None if row_scale is None else np.ascontiguousarray(row_scale, dtype=np.float32)
    bt = None if block_table is None else np.ascontiguousarray(block_table, dtype=np.int32)
    wv = None if w_uv is None else _arr(w_uv, wd)
    dv = 0 if wv is None else int(wv.shape[1])
    if seq_stride is None:
        seq_stride = int(seq_lens.max()) if B else 0
    P = _Problem(B, H, int(d_nope), dr, dl, dv, float(scale) if scale else 0.0, None, None, 0,
                 None, _ptr(wv), wd, _ptr(rows), _ptr(rs), cd, int(page_size), int(seq_stride),
                 _ptr(bt), 0 if bt is None else int(bt.shape[1]), _ptr(seq_lens), int(bool(ring)))
    if sel is None:
        n = B * H
        sb = sh = None
    else:
        sel = list(sel)
        n = len(sel)
        sb = np.ascontiguousarray([x[0] for x in sel], dtype=np.int32)
        sh = np.ascontiguousarray([x[1] for x in sel], dtype=np.int32)
    tb = None if t_begin is None else np.ascontiguousarray(t_begin, dtype=np.int32)
    te = None if t_end is None else np.ascontiguousarray(t_end, dtype=np.int32)
    u = np.zeros((n, dl), dtype=np.float64)
    lse = np.zeros(n, dtype=np.float64)
    o = None if wv is None else np.zeros((n, dv), dtype=np.float64)
    rc = lib().oracle_absorbed_decode(C.byref(P), _ptr(q_abs), qd, _ptr(qs), _ptr(sb), _ptr(sh),
                                      n, _ptr(tb), _ptr(te), _ptr(u), _ptr(lse), _ptr(o))
    if rc != 0:
        raise ValueError(f"oracle_absorbed_decode failed: {rc}")
    return u, lse, o


def quantize_e4m3_rows(x):
    """E4M3 codes and one fp32 factor per row of the binary32 array x [..., w]
    (the E4M3 cache rule).  Returns (codes uint8 like x, scale float32 x.shape[:-1])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    w = x.shape[-1]
    n = x.size // w
    codes = np.zeros(x.shape, dtype=np.uint8)
    scale = np.zeros(x.shape[:-1], dtype=np.float32)
    rc = lib().oracle_quantize_e4m3_rows(n, w, _ptr(x), _ptr(codes), _ptr(scale))
    if rc != 0:
        raise ValueError(f"oracle_quantize_e4m3_rows failed: {rc}")
    return codes, scale


def absorb_q_fp8(q_nope, q_rope, q_dtype, w_uk, w_dtype):
    """The absorbed query in E4M3 with one factor per (b, h): the float64
    absorbed rows rounded to binary32, then quantize_e4m3_rows.  Returns
    (codes [B, H, d_latent + d_rope] uint8, scale [B, H] float32)."""
    qa = absorb_q(q_nope, q_rope, q_dtype, w_uk, w_dtype)
    return quantize_e4m3_rows(qa.astype(np.float32))


def absorb_q(q_nope, q_rope, q_dtype, w_uk, w_dtype):
    """q_abs [B, H, d_latent + d_rope] float64."""
    qd, wd = _dt(q_dtype), _dt(w_dtype)
    q_nope, q_rope, w_uk = _arr(q_nope, qd), _arr(q_rope, qd), _arr(w_uk, wd)
    B, H, dn = q_nope.shape
    dr, dl = q_rope.shape[2], w_uk.shape[2]
    out = np.zeros((B, H, dl + dr), dtype=np.float64)
    rc = lib().oracle_absorb_q(B, H, dn, dr, dl, _ptr(q_nope), _ptr(q_rope), qd, _ptr(w_uk),
                               wd, _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_absorb_q failed: {rc}")
    return out


def combine(u_part, lse_part):
    """u_part [B, S, H, D], lse_part [B, S, H] (float64) -> (u [B, H, D], lse [B, H])."""
    u_part = np.ascontiguousarray(u_part, dtype=np.float64)
    lse_part = np.ascontiguousarray(lse_part, dtype=np.float64)
    B, S, H, D = u_part.shape
    u = np.zeros((B, H, D), dtype=np.float64)
    lse = np.zeros((B, H), dtype=np.float64)
    rc = lib().oracle_combine(B, S, H, D, _ptr(u_part), _ptr(lse_part), _ptr(u), _ptr(lse))
    if rc != 0:
        raise ValueError(f"oracle_combine failed: {rc}")
    return u, lse


def cache_append(c_kv, k_r, src_dtype, positions, rows, cache_dtype, row_scale=None,
                 page_size=0, seq_stride=0, block_table=None, ring=False):
    """Write one token per sequence into the cache arrays (modified in place).

    c_kv [B, d_latent], k_r [B, d_rope] stored bits in src_dtype ("f32" or
    "bf16"); rows [n_rows, d_latent + d_rope] stored bits in cache_dtype;
    row_scale [n_rows] float32 for "fp8"; positions [B] int32 (negative or
    past the capacity: skipped; a ring (contiguous, ring=True) writes token t
    into row t mod seq_stride of its sequence)."""
    sd, cd = _dt(src_dtype), _dt(cache_dtype)
    c_kv, k_r = _arr(c_kv, sd), _arr(k_r, sd)
    B, dl = c_kv.shape
    dr = k_r.shape[1]
    pos = np.ascontiguousarray(positions, dtype=np.int32)
    assert rows.flags.c_contiguous and rows.dtype == _NP[cd]
    if row_scale is not None:
        assert row_scale.flags.c_contiguous and row_scale.dtype == np.float32
    bt = None if block_table is None else np.ascontiguousarray(block_table, dtype=np.int32)
    max_pages = 0 if bt is None else bt.shape[1]
    rc = lib().oracle_cache_append(B, dl, dr, _ptr(c_kv), _ptr(k_r), sd, _ptr(pos), _ptr(rows),
                                   cd, _ptr(row_scale), int(page_size), int(seq_stride), _ptr(bt),
                                   max_pages, int(bool(ring)))
    if rc != 0:
        raise ValueError(f"oracle_cache_append failed: {rc}")


def gqa_decode(q, k, v, dtype, seq_lens, scale=0.0):
    """Grouped-query attention decode.  q [B, H, d_qk]; k [B, H_kv, stride,
    d_qk], v [B, H_kv, stride, d_v] (stored bits in dtype), H a multiple of
    H_kv, query head h reading key/value head h // (H / H_kv); seq_lens [B]
    -> (o [B, H, d_v], lse [B, H]) float64."""
    d = _dt(dtype)
    q, k, v = _arr(q, d), _arr(k, d), _arr(v, d)
    B, H, dq = q.shape
    Hkv, stride, dv = k.shape[1], k.shape[2], v.shape[3]
    assert k.shape == (B, Hkv, stride, dq) and v.shape[:3] == (B, Hkv, stride)
    lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    o = np.zeros((B, H, dv), dtype=np.float64)
    lse = np.zeros((B, H), dtype=np.float64)
    rc = lib().oracle_gqa_decode(B, H, Hkv, dq, dv, _ptr(q), _ptr(k), _ptr(v), d, _ptr(lens),
                                 stride, float(scale), _ptr(o), _ptr(lse))
    if rc != 0:
        raise ValueError(f"oracle_gqa_decode failed: {rc}")
    return o, lse


def ring_grow(seq_lens, src, src_cap, dst_cap, src_scale=None):
    """Move each sequence's live window from a ring of src_cap rows per
    sequence (src [B*src_cap, W], any dtype) into a new ring of dst_cap rows
    (token t to row t mod dst_cap).  Returns (dst, dst_scale or None); rows
    the window does not reach are zero."""
    lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    B = lens.shape[0]
    src = np.ascontiguousarray(src)
    W = src.shape[1]
    dst = np.zeros((B * dst_cap, W), dtype=src.dtype)
    ss = None if src_scale is None else np.ascontiguousarray(src_scale, dtype=np.float32)
    ds = None if ss is None else np.zeros(B * dst_cap, dtype=np.float32)
    rc = lib().oracle_ring_grow(B, W * src.dtype.itemsize, _ptr(lens), _ptr(src), _ptr(ss),
                                int(src_cap), _ptr(dst), _ptr(ds), int(dst_cap))
    if rc != 0:
        raise ValueError(f"oracle_ring_grow failed: {rc}")
    return dst, ds


def mha_decode(q, k, v, dtype, seq_lens, scale=0.0):
    """Textbook multi-head attention decode over a per-head cache.
    q [B, H, d_qk], k [B, H, stride, d_qk], v [B, H, stride, d_v] (stored bits
    in dtype), seq_lens [B] -> (o [B, H, d_v], lse [B, H]) float64."""
    d = _dt(dtype)
    q, k, v = _arr(q, d), _arr(k, d), _arr(v, d)
    B, H, dq = q.shape
    stride, dv = k.shape[2], v.shape[3]
    assert k.shape == (B, H, stride, dq) and v.shape[:3] == (B, H, stride)
    lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    o = np.zeros((B, H, dv), dtype=np.float64)
    lse = np.zeros((B, H), dtype=np.float64)
    rc = lib().oracle_mha_decode(B, H, dq, dv, _ptr(q), _ptr(k), _ptr(v), d, _ptr(lens), stride,
                                 float(scale), _ptr(o), _ptr(lse))
    if rc != 0:
        raise ValueError(f"oracle_mha_decode failed: {rc}")
    return o, lse


def rope(x, dtype, positions, base=10000.0):
    """Decoupled RoPE of x [B, H, d_r] (stored bits in dtype) at positions [B]
    (int32) -> float64 [B, H, d_r]."""
    d = _dt(dtype)
    x = _arr(x, d)
    B, H, dr = x.shape
    pos = np.ascontiguousarray(positions, dtype=np.int32)
    out = np.zeros((B, H, dr), dtype=np.float64)
    rc = lib().oracle_rope(B, H, dr, _ptr(x), d, _ptr(pos), float(base), _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_rope failed: {rc}")
    return out


def rope_inv_freq(d_r=64, base=10000.0) -> np.ndarray:
    f = np.zeros(d_r // 2, dtype=np.float32)
    lib().oracle_rope_inv_freq(d_r, float(base), _ptr(f))
    return f


def encode_e4m3(y: float) -> int:
    """The E4M3 code nearest to the binary32 value y (|y| <= 448)."""
    return int(lib().oracle_encode_e4m3(float(y)))


def up_proj(u, w_uv, w_dtype):
    """u [B, H, d_latent] float64, W_UV [H, d_v, d_latent] -> o [B, H, d_v]."""
    wd = _dt(w_dtype)
    u = np.ascontiguousarray(u, dtype=np.float64)
    w_uv = _arr(w_uv, wd)
    B, H, dl = u.shape
    dv = w_uv.shape[1]
    o = np.zeros((B, H, dv), dtype=np.float64)
    rc = lib().oracle_up_proj(B, H, dv, dl, _ptr(u), _ptr(w_uv), wd, _ptr(o))
    if rc != 0:
        raise ValueError(f"oracle_up_proj failed: {rc}")
    return o


def decode_array(a, dtype) -> np.ndarray:
    """Decode stored bits to float64 with the oracle's own decoder."""
    d = _dt(dtype)
    a = _arr(a, d)
    out = np.empty(a.shape, dtype=np.float64)
    lib().oracle_decode_array(_ptr(a), d, a.size, _ptr(out))
    return out


def mla_cache_bytes_per_token(d_latent, d_rope, elem_bytes, scale_bytes=0) -> int:
    return int(lib().oracle_mla_cache_bytes_per_token(d_latent, d_rope, elem_bytes,
                                                      scale_bytes))


def mha_cache_bytes(layers, seq_len, heads, head_dim, elem_bytes) -> int:
    return int(lib().oracle_mha_cache_bytes(layers, seq_len, heads, head_dim, elem_bytes))


def num_threads() -> int:
    return int(lib().oracle_num_threads())

"""The C ABI without a GPU: the library loads, exports every function that
include/mla.h declares, and rejects bad arguments on the host with the
documented status before anything is launched.  Pointers here are fake,
never-dereferenced addresses; no call reaches a kernel."""

import ctypes as C
import os
import re

import pytest

import mla_latent_kv_15_amd as mla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")

OK, E_ARG, E_DTYPE, E_SHAPE, E_ALIGN, E_HIP, E_UNSUP, E_SCRATCH = range(8)
F32, BF16, FP8 = mla.MLA_F32, mla.MLA_BF16, mla.MLA_FP8_E4M3
P = 0x10000  # a fake, 64 KiB-aligned "device" address: never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_\w+)\s*\(", text)))


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("mla_absorb_q", "mla_decode", "mla_combine", "mla_up_proj", "mla_status_str"):
        assert n in names


def test_every_declared_symbol_is_exported():
    L = mla.lib()
    for n in declared_functions():
        assert hasattr(L, n), n
    assert set(declared_functions()) == set(mla.EXPORTED)


def test_status_strings():
    for s in range(8):
        assert mla.status_str(s) and mla.status_str(s) != "unknown status"
    assert mla.status_str(99) == "unknown status"
    assert mla.lib().mla_version() >= 100


def dims(h=128, dn=128, dr=64, dl=512, dv=128, scale=0.0):
    return mla.Dims(h, dn, dr, dl, dv, scale)


def cache(dtype=BF16, rows=P, row_scale=None, page_size=0, seq_stride=4096, block_table=None,
          max_pages=0, seq_lens=P, max_seq_len=4096, ring=0):
    return mla.CacheDesc(dtype, rows, row_scale, page_size, seq_stride, block_table, max_pages,
                         seq_lens, max_seq_len, ring)


def decode(d=None, B=2, q=P, q_dt=BF16, q_scale=None, c=None, S=4, u=P, u_dt=F32, lse=P):
    d = d or dims()
    c = c or cache()
    return mla.lib().mla_decode(C.byref(d), B, q, q_dt, q_scale, C.byref(c), S, u, u_dt, lse,
                                None)


def test_decode_validation():
    L = mla.lib()
    assert decode(B=0, q=None, u=None, lse=None) == OK  # nothing to do, nothing launched
    assert L.mla_decode(None, 1, P, BF16, None, C.byref(cache()), 1, P, F32, P, None) == E_ARG
    assert L.mla_decode(C.byref(dims()), 1, P, BF16, None, None, 1, P, F32, P, None) == E_ARG
    assert decode(q=None) == E_ARG
    assert decode(u=None) == E_ARG
    assert decode(lse=None) == E_ARG
    assert decode(c=cache(rows=None)) == E_ARG
    assert decode(c=cache(seq_lens=None)) == E_ARG
    assert decode(B=-1) == E_ARG
    assert decode(S=0) == E_ARG
    assert decode(S=1025) == E_ARG
    assert decode(q_dt=7) == E_ARG
    assert decode(d=dims(dl=256)) == E_SHAPE
    assert decode(d=dims(dr=32)) == E_SHAPE
    assert decode(d=dims(h=0)) == E_ARG
    assert decode(d=dims(h=48)) == E_SHAPE  # MFMA paths need h % 32 == 0
    assert decode(d=dims(scale=float("nan"))) == E_ARG
    assert decode(c=cache(page_size=32)) == E_SHAPE
    assert decode(c=cache(seq_stride=100)) == E_ARG  # stride below the longest sequence
    assert decode(c=cache(max_seq_len=-1)) == E_ARG
    # paged: block table present and wide enough
    assert decode(c=cache(page_size=64, block_table=None, max_pages=64)) == E_ARG
    assert decode(c=cache(page_size=64, block_table=P, max_pages=63)) == E_ARG
    # dtype pairs
    assert decode(q_dt=F32) == E_DTYPE  # bf16 cache with fp32 q_abs
    assert decode(c=cache(dtype=F32), q_dt=BF16) == E_DTYPE
    assert decode(u_dt=FP8) == E_DTYPE
    assert decode(c=cache(dtype=FP8)) == E_ARG  # fp8 cache without row scales
    assert decode(c=cache(dtype=BF16, row_scale=P)) == E_ARG  # scales on a bf16 cache
    assert decode(q_scale=P) == E_ARG  # q scales with a bf16 query
    # an E4M3 query: an E4M3 cache only, with its factors
    f8 = cache(dtype=FP8, row_scale=P)
    assert decode(q_dt=FP8, q_scale=None, c=f8) == E_ARG
    assert decode(q_dt=FP8, q_scale=P) == E_DTYPE  # bf16 cache
    assert decode(q_dt=FP8, q_scale=P, c=cache(dtype=F32)) == E_DTYPE
    # alignment
    assert decode(c=cache(rows=P + 8)) == E_ALIGN
    assert decode(q=P + 2) == E_ALIGN
    assert decode(u=P + 4) == E_ALIGN


def test_absorb_validation():
    L = mla.lib()
    d = dims()

    def absorb(B=2, qn=P, qr=P, q_dt=BF16, w=P, w_dt=BF16, out=P, out_dt=BF16, scale=None, dd=d):
        return L.mla_absorb_q(C.byref(dd), B, qn, qr, q_dt, w, w_dt, out, out_dt, scale, None)

    assert absorb(B=0, qn=None, qr=None, w=None, out=None) == OK
    assert absorb(qn=None) == E_ARG
    assert absorb(w=None) == E_ARG
    assert absorb(q_dt=FP8) == E_DTYPE
    assert absorb(out_dt=FP8, scale=None) == E_ARG
    assert absorb(out_dt=BF16, scale=P) == E_ARG
    # the E4M3 output needs bf16 inputs and d_nope <= 128 (host checks, nothing launched)
    assert absorb(out_dt=FP8, scale=P, q_dt=F32) == E_UNSUP
    assert absorb(out_dt=FP8, scale=P, w_dt=F32) == E_UNSUP
    assert absorb(out_dt=FP8, scale=P, dd=dims(dn=192)) == E_UNSUP
    assert absorb(out_dt=FP8, scale=P, qn=P + 2) == E_UNSUP
    assert absorb(dd=dims(dn=300)) == E_SHAPE
    assert absorb(out=P + 2) == E_ALIGN


def test_combine_and_up_proj_validation():
    L = mla.lib()
    d = dims()
    assert L.mla_combine(C.byref(d), 0, 4, None, F32, None, None, F32, None, None) == OK
    assert L.mla_combine(C.byref(d), 2, 0, P, F32, P, P, F32, None, None) == E_ARG
    assert L.mla_combine(C.byref(d), 2, 4, None, F32, P, P, F32, None, None) == E_ARG
    assert L.mla_combine(C.byref(d), 2, 4, P, FP8, P, P, F32, None, None) == E_DTYPE
    assert L.mla_combine(C.byref(d), 2, 4, P + 4, F32, P, P, F32, None, None) == E_ALIGN
    assert L.mla_up_proj(C.byref(d), 0, None, F32, None, F32, None, F32, None) == OK
    assert L.mla_up_proj(C.byref(d), 2, P, F32, None, F32, P, F32, None) == E_ARG
    assert L.mla_up_proj(C.byref(d), 2, P, FP8, P, F32, P, F32, None) == E_DTYPE
    assert L.mla_up_proj(C.byref(dims(dv=512)), 2, P, F32, P, F32, P, F32, None) == E_SHAPE


def test_combine_up_proj_validation():
    L = mla.lib()
    d = dims()

    def cu(B=2, S=4, up=P, p_dt=BF16, lse=P, w=P, w_dt=BF16, o=P, o_dt=BF16, u=None, l=None, dd=d):
        return L.mla_combine_up_proj(C.byref(dd), B, S, up, p_dt, lse, w, w_dt, o, o_dt, u, l, None)

    assert cu(B=0, up=None, lse=None, w=None, o=None) == OK
    assert cu(S=0) == E_ARG
    assert cu(S=1025) == E_ARG
    assert cu(up=None) == E_ARG
    assert cu(lse=None) == E_ARG
    assert cu(w=None) == E_ARG
    assert cu(o=None) == E_ARG
    assert cu(p_dt=9) == E_ARG
    assert cu(p_dt=FP8) == E_DTYPE
    assert cu(o_dt=FP8) == E_DTYPE
    assert cu(w_dt=F32) == E_DTYPE  # bf16 W_UV only
    assert cu(dd=dims(dv=120)) == E_SHAPE  # d_v % 16
    assert cu(up=P + 4) == E_ALIGN
    assert cu(w=P + 2) == E_ALIGN
    assert cu(u=P + 2) == E_ALIGN


@pytest.mark.parametrize("L,S,expect", [(0, 4, 0), (1, 1, 32), (2048, 8, 256), (32768, 64, 512),
                                         (131072, 256, 512), (16384, 32, 512), (100, 3, 64),
                                         (33, 1, 64)])
def test_split_chunk_rule(L, S, expect):
    assert mla.split_chunk(L, S) == expect
    if L:
        assert expect % mla.TILE_TOKENS == 0 and expect * S >= L


def test_cache_append_validation():
    L = mla.lib()

    def ap(B=2, ckv=P, kr=P, src=BF16, pos=P, c=None, d=None):
        c = c if c is not None else cache()
        return L.mla_cache_append(C.byref(d or dims()), B, ckv, kr, src, pos, C.byref(c), None)

    assert ap(B=0, ckv=None, kr=None, pos=None) == OK
    assert ap(B=-1) == E_ARG
    assert ap(ckv=None) == E_ARG
    assert ap(kr=None) == E_ARG
    assert ap(pos=None) == E_ARG
    assert ap(c=cache(rows=None)) == E_ARG
    assert ap(src=9) == E_ARG
    assert ap(src=FP8) == E_DTYPE
    assert ap(c=cache(dtype=FP8)) == E_ARG                 # fp8 needs row_scale
    assert ap(c=cache(dtype=BF16, row_scale=P)) == E_ARG   # only fp8 has one
    assert ap(c=cache(seq_stride=0)) == E_ARG
    assert ap(c=cache(page_size=32, block_table=P, max_pages=4)) == E_SHAPE
    assert ap(c=cache(page_size=64, block_table=None, max_pages=4)) == E_ARG
    assert ap(c=cache(page_size=64, block_table=P, max_pages=0)) == E_ARG
    assert ap(c=cache(rows=P + 8)) == E_ALIGN
    assert ap(d=dims(dl=256)) == E_SHAPE


def test_absorb_q_rope_validation():
    L = mla.lib()

    def ar(B=2, qn=P, qr=P, q_dt=BF16, w=P, w_dt=BF16, pos=P, base=10000.0, qa=P, qa_dt=BF16):
        return L.mla_absorb_q_rope(C.byref(dims()), B, qn, qr, q_dt, w, w_dt, pos, base, qa, qa_dt,
                                   None)

    assert ar(B=0, qn=None, qr=None, w=None, pos=None, qa=None) == OK
    assert ar(pos=None) == E_ARG
    assert ar(base=1.0) == E_ARG
    assert ar(base=float("inf")) == E_ARG
    assert ar(base=float("nan")) == E_ARG
    assert ar(B=0, base=0.5) == E_ARG
    assert ar(qn=None) == E_ARG
    assert ar(q_dt=FP8) == E_DTYPE
    assert ar(qa_dt=FP8) == E_ARG  # an fp8 q_abs needs a scale this call does not take
    assert ar(qa=P + 8) == E_ALIGN


def test_mha_decode_validation():
    L = mla.lib()

    def mh(B=2, H=128, D=128, q=P, k=P, v=P, dt=BF16, lens=P, stride=4096, maxl=4096, sc=0.0,
           o=P, o_dt=BF16, lse=None):
        return L.mla_mha_decode(B, H, D, q, k, v, dt, lens, stride, maxl, sc, o, o_dt, lse, None)

    assert mh(B=0, q=None, k=None, v=None, lens=None, o=None) == OK
    assert mh(B=-1) == E_ARG
    assert mh(H=0) == E_ARG
    assert mh(D=64) == E_SHAPE
    assert mh(q=None) == E_ARG
    assert mh(k=None) == E_ARG
    assert mh(lens=None) == E_ARG
    assert mh(o=None) == E_ARG
    assert mh(stride=100, maxl=200) == E_ARG
    assert mh(maxl=-1) == E_ARG
    assert mh(sc=float("nan")) == E_ARG
    assert mh(dt=F32) == E_DTYPE
    assert mh(o_dt=FP8) == E_DTYPE
    assert mh(dt=7) == E_ARG
    assert mh(k=P + 2) == E_ALIGN


def test_decode_multi_validation():
    L = mla.lib()

    def dm(B=2, ql=4, q=P, q_dt=BF16, c=None, S=4, u=P, u_dt=BF16, lse=P):
        c = c if c is not None else cache()
        return L.mla_decode_multi(C.byref(dims()), B, ql, q, q_dt, C.byref(c), S, u, u_dt, lse,
                                  None)

    assert dm(B=0, q=None, u=None, lse=None) == OK
    assert dm(ql=0) == E_ARG
    assert dm(ql=17) == E_ARG
    assert dm(q=None) == E_ARG
    assert dm(S=0) == E_ARG
    assert dm(q_dt=F32) == E_DTYPE          # bf16 cache, fp32 queries
    assert dm(u_dt=FP8) == E_DTYPE
    assert dm(c=cache(dtype=FP8)) == E_ARG  # fp8 cache without row scales
    assert dm(u=P + 4) == E_ALIGN


def test_decode_ex_kernel_choice_validation():
    """mla_decode_ex: the kernel argument is checked on the host before any
    launch; the balanced partition's limits, the retired values, unknown ones."""
    L = mla.lib()

    def dx(kernel, h=128, c=None, B=2, ql=1, S=4):
        c = c if c is not None else cache()
        return L.mla_decode_ex(C.byref(dims(h=h)), B, ql, P, BF16, C.byref(c), S, P, BF16, P,
                               kernel, None)

    assert dx(mla.KERNEL_H64, B=0) == OK
    assert dx(5) == E_ARG
    # the balanced partition: bf16 cache, at least 2 splits, at most 512 rows
    BAL = mla.KERNEL_H64_BALANCED
    assert dx(BAL, c=cache(dtype=FP8, row_scale=P)) == E_UNSUP
    assert dx(BAL, S=1) == E_UNSUP
    assert dx(BAL, B=513) == E_UNSUP
    assert dx(BAL, B=128, ql=5) == E_UNSUP
    assert dx(BAL, B=0) == OK
    assert dx(-1) == E_ARG
    # values 2 and 3: the retired 128-head workgroups
    assert dx(2) == E_UNSUP
    assert dx(3) == E_UNSUP
    assert dx(mla.KERNEL_H64, ql=0) == E_ARG
    assert dx(mla.KERNEL_H64, ql=17) == E_ARG


def noalloc(d=None, B=2, q=P, q_dt=BF16, c=None, S=4, w=P, w_dt=BF16, o=P, o_dt=BF16, u=None,
            lse=None):
    d = d or dims()
    c = c or cache()
    return mla.lib().mla_decode_combine_up_proj_noalloc(C.byref(d), B, q, q_dt, C.byref(c), S, w,
                                                        w_dt, o, o_dt, u, lse, None)


def test_noalloc_validation_before_any_launch():
    """The no-allocation decode + tail checks its arguments like mla_decode and
    mla_combine_up_proj, and refuses a request beyond its static scratch (B *
    num_splits * heads > 65536 rows) before touching the device."""
    assert noalloc(B=0) == OK
    assert noalloc(q=None) == E_ARG
    assert noalloc(w=None) == E_ARG
    assert noalloc(o=None) == E_ARG
    assert noalloc(S=0) == E_ARG
    assert noalloc(S=1025) == E_ARG
    assert noalloc(w_dt=F32) == E_DTYPE
    assert noalloc(o_dt=FP8) == E_DTYPE
    assert noalloc(d=dims(dv=120)) == E_SHAPE
    assert noalloc(w=P + 8) == E_ALIGN
    assert noalloc(B=65, S=8) == E_SCRATCH          # 66,560 rows
    assert noalloc(B=1, S=1024, d=dims(h=128)) == E_SCRATCH  # 131,072 rows
    assert noalloc(B=513, S=1) == E_SCRATCH


def test_ring_cache_validation():
    """A ring is contiguous; its lengths may exceed its capacity; a multi-token
    decode over a ring is refused (earlier query tokens would need rows the
    ring overwrote) before any launch."""
    assert decode(c=cache(ring=2)) == E_ARG
    assert decode(c=cache(ring=1, page_size=64, block_table=P, max_pages=64)) == E_ARG
    assert decode(c=cache(ring=1, seq_stride=0)) == E_ARG
    assert decode(c=cache(ring=0, seq_stride=1024, max_seq_len=4096)) == E_ARG
    d = dims()
    multi = mla.lib().mla_decode_multi(C.byref(d), 2, 2, P, BF16,
                                       C.byref(cache(ring=1, seq_stride=1024, max_seq_len=4096)),
                                       4, P, F32, P, None)
    assert multi == E_UNSUP
    src, dst = cache(ring=1, seq_stride=256), cache(ring=1, seq_stride=512)
    L = mla.lib()
    assert L.mla_cache_ring_grow(0, C.byref(src), C.byref(dst), None) == OK
    assert L.mla_cache_ring_grow(2, C.byref(src), C.byref(cache(ring=0)), None) == E_ARG
    assert L.mla_cache_ring_grow(2, None, C.byref(dst), None) == E_ARG
    assert L.mla_cache_ring_grow(2, C.byref(src), C.byref(cache(ring=1, dtype=F32)), None) == E_DTYPE
    assert L.mla_cache_ring_grow(2, C.byref(src), C.byref(cache(ring=1, rows=P + 8)), None) == E_ALIGN
    fp8 = cache(ring=1, dtype=FP8, row_scale=P)
    assert L.mla_cache_ring_grow(2, C.byref(fp8), C.byref(cache(ring=1, dtype=FP8)), None) == E_ARG


def test_prefill_validation():
    L = mla.lib()
    d = dims()
    c = cache(seq_stride=4096, max_seq_len=4096)

    def rb(d=d, B=2, c=c, frm=None, wk=P, wv=P, w_dt=BF16, k=P, vt=P, S=4096):
        return L.mla_prefill_rebuild_kv(C.byref(d), B, C.byref(c), frm, wk, wv, w_dt, k, vt, S, None)

    def at(d=d, B=2, QL=64, ql=P, q=P, q_dt=BF16, k=P, vt=P, S=4096, sl=P, msl=4096, o=P,
           o_dt=BF16):
        return L.mla_prefill_attn(C.byref(d), B, QL, ql, q, q_dt, k, vt, S, sl, msl, o, o_dt,
                                  None, None)

    assert rb(B=0) == OK and at(B=0) == OK and at(QL=0) == OK
    assert rb(wk=None) == E_ARG and rb(k=None) == E_ARG and rb(c=cache(rows=None)) == E_ARG
    assert rb(S=4064) == E_ARG and rb(S=4100) == E_ARG          # < max_seq_len, not x32
    assert rb(d=dims(dn=64)) == E_SHAPE and rb(d=dims(dv=64)) == E_SHAPE
    assert rb(w_dt=F32) == E_DTYPE and rb(c=cache(dtype=F32)) == E_DTYPE
    assert rb(c=cache(ring=1, seq_stride=4096)) == E_UNSUP
    assert rb(k=P + 8) == E_ALIGN
    assert at(q=None) == E_ARG and at(ql=None) == E_ARG and at(S=4000) == E_ARG
    assert at(q_dt=F32) == E_DTYPE and at(o_dt=FP8) == E_DTYPE
    assert at(d=dims(dn=192)) == E_SHAPE and at(o=P + 4) == E_ALIGN


def test_stream_probe_validation_before_any_launch():
    """mla_stream_probe refuses bad arguments on the host: NULL pointers, no
    workgroups or tiles, an odd paired count, a misaligned source, a source
    shorter than the tiles it would stream"""
    L = mla.lib()

    def sp(src=P, nbytes=1 << 30, wg=256, tiles=100, paired=1, sink=P):
        return L.mla_stream_probe(src, nbytes, wg, tiles, paired, sink, None)

    assert sp(src=None) == E_ARG
    assert sp(sink=None) == E_ARG
    assert sp(wg=0) == E_ARG
    assert sp(tiles=0) == E_ARG
    assert sp(wg=255) == E_ARG
    assert sp(src=P + 8) == E_ALIGN
    assert sp(nbytes=128 * 100 * 36864 - 1) == E_SHAPE
    assert sp(nbytes=256 * 100 * 36864 - 1, paired=0) == E_SHAPE

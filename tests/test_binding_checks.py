"""The Python binding rejects, before anything reaches the C library, every
buffer whose device, dtype or shape differs from what the call implies (the
kernels index buffers by B, S, heads and the widths, so a short buffer would be
read or written out of bounds on the GPU).  CPU tensors stand in for device
buffers: with the right shapes they fail only the device check, with a wrong
shape they fail the shape check first."""

import pytest
import torch

import mla_latent_kv_15_amd as mla

B, S, H, DN, DV = 3, 2, 16, 128, 128
GEO = mla.Geometry(heads=H)


def t(*shape, dtype=torch.bfloat16):
    return torch.zeros(*shape, dtype=dtype)


@pytest.fixture(autouse=True)
def no_c_calls(monkeypatch):
    """Any call that got past the checks would reach this stub and fail."""
    class Stub:
        def __getattr__(self, name):
            raise AssertionError(f"{name} reached the C library")
    monkeypatch.setattr(mla, "lib", lambda: Stub())


def good_cache(B=B, L=100, stride=128, paged=False, fp8=False):
    rows_dt = torch.uint8 if fp8 else torch.bfloat16
    if paged:
        mp = 2
        return mla.Cache(rows=t(B * mp * 64, 576, dtype=rows_dt),
                         seq_lens=t(B, dtype=torch.int32), max_seq_len=L,
                         row_scale=t(B * mp * 64, dtype=torch.float32) if fp8 else None,
                         block_table=t(B, mp, dtype=torch.int32), page_size=64)
    return mla.Cache(rows=t(B * stride, 576, dtype=rows_dt), seq_lens=t(B, dtype=torch.int32),
                     max_seq_len=L, row_scale=t(B * stride, dtype=torch.float32) if fp8 else None,
                     seq_stride=stride)


def raises_shape(fn, *a, **k):
    with pytest.raises(ValueError, match="shape|rows|stride|pages|block_table"):
        fn(*a, **k)


def raises_device(fn, *a, **k):
    with pytest.raises(ValueError, match="on the GPU"):
        fn(*a, **k)


def test_absorb():
    args = dict(q_nope=t(B, H, DN), q_rope=t(B, H, 64), w_uk=t(H, DN, 512), q_abs=t(B, H, 576))
    raises_device(mla.mla_absorb_q, GEO, **args)
    for k, bad in [("q_rope", t(B, H, 63)), ("w_uk", t(H, DN, 511)), ("w_uk", t(H - 1, DN, 512)),
                   ("q_abs", t(B - 1, H, 576)), ("q_abs", t(B, H, 512))]:
        raises_shape(mla.mla_absorb_q, GEO, **{**args, k: bad})
    raises_shape(mla.mla_absorb_q, GEO, **args, q_abs_scale=t(B, H - 1, dtype=torch.float32))
    with pytest.raises(TypeError):
        mla.mla_absorb_q(GEO, **args, q_abs_scale=t(B, H, dtype=torch.bfloat16))
    pos = t(B, dtype=torch.int32)
    raises_device(mla.mla_absorb_q_rope, GEO, args["q_nope"], args["q_rope"], args["w_uk"], pos,
                  args["q_abs"])
    raises_shape(mla.mla_absorb_q_rope, GEO, args["q_nope"], args["q_rope"], args["w_uk"],
                 t(B + 1, dtype=torch.int32), args["q_abs"])


@pytest.mark.parametrize("paged,fp8", [(False, False), (True, False), (False, True)])
def test_decode(paged, fp8):
    q = t(B, H, 576)
    up, lp = t(B, S, H, 512), t(B, S, H, dtype=torch.float32)
    c = good_cache(paged=paged, fp8=fp8)
    raises_device(mla.mla_decode, GEO, q, c, S, up, lp)
    raises_shape(mla.mla_decode, GEO, q, c, S + 1, up, lp)  # split count vs partials
    raises_shape(mla.mla_decode, GEO, q, c, S, t(B, S, H, 256), lp)
    raises_shape(mla.mla_decode, GEO, q, c, S, up, t(B, S, H - 1, dtype=torch.float32))
    raises_shape(mla.mla_decode, GEO, t(B, H, 575), c, S, up, lp)
    bad = good_cache(B=B + 1, paged=paged, fp8=fp8)  # seq_lens / block table for another batch
    raises_shape(mla.mla_decode, GEO, q, bad, S, up, lp)
    if paged:
        short = good_cache(paged=True, L=200)  # 2 pages of 64 < 200 tokens
        raises_shape(mla.mla_decode, GEO, q, short, S, up, lp)
    else:
        short = good_cache(L=200)  # stride 128 < 200
        raises_shape(mla.mla_decode, GEO, q, short, S, up, lp)
        c2 = good_cache()
        c2.rows = t(B * 128 - 29, 576)  # last sequence cut short
        raises_shape(mla.mla_decode, GEO, q, c2, S, up, lp)
    if fp8:
        c3 = good_cache(fp8=True)
        c3.row_scale = t(10, dtype=torch.float32)
        raises_shape(mla.mla_decode, GEO, q, c3, S, up, lp)


def test_decode_multi_and_ex():
    QL = 3
    q = t(B, QL, H, 576)
    up, lp = t(B, QL, S, H, 512), t(B, QL, S, H, dtype=torch.float32)
    c = good_cache()
    raises_device(mla.mla_decode_multi, GEO, q, c, S, up, lp)
    raises_device(mla.mla_decode_ex, GEO, q, c, S, up, lp)
    raises_shape(mla.mla_decode_multi, GEO, q, c, S, t(B, S, H, 512), lp)
    raises_shape(mla.mla_decode_ex, GEO, q, c, S, up, t(B, QL, S + 1, H, dtype=torch.float32))
    raises_shape(mla.mla_decode_ex, GEO, t(B, H, 576), c, S, up, lp)


def test_tail():
    up, lp = t(B, S, H, 512), t(B, S, H, dtype=torch.float32)
    u, lse, o, w = t(B, H, 512), t(B, H, dtype=torch.float32), t(B, H, DV), t(H, DV, 512)
    raises_device(mla.mla_combine, GEO, up, lp, u, lse)
    raises_shape(mla.mla_combine, GEO, up, lp, t(B, H, 256), lse)
    raises_shape(mla.mla_combine, GEO, up, t(B, S - 1, H, dtype=torch.float32), u, lse)
    raises_shape(mla.mla_combine, GEO, up, lp, u, t(B, H + 1, dtype=torch.float32))
    raises_device(mla.mla_up_proj, GEO, u, w, o)
    raises_shape(mla.mla_up_proj, GEO, u, t(H, DV - 1, 512), o)
    raises_shape(mla.mla_up_proj, GEO, u, w, t(B - 1, H, DV))
    raises_device(mla.mla_combine_up_proj, GEO, up, lp, w, o, u, lse)
    raises_shape(mla.mla_combine_up_proj, GEO, up, lp, w, t(B, H, DV // 2))
    raises_shape(mla.mla_combine_up_proj, GEO, up, lp, w, o, t(B, H - 1, 512))
    raises_shape(mla.mla_combine_up_proj, GEO, up, lp, t(H, DV, 256), o)


def test_append_and_mha():
    c = good_cache()
    ckv, kr, pos = t(B, 512), t(B, 64), t(B, dtype=torch.int32)
    raises_device(mla.mla_cache_append, GEO, ckv, kr, pos, c)
    raises_shape(mla.mla_cache_append, GEO, ckv, t(B, 32), pos, c)
    raises_shape(mla.mla_cache_append, GEO, ckv, kr, t(B - 1, dtype=torch.int32), c)
    raises_shape(mla.mla_cache_append, GEO, ckv, kr, pos, good_cache(B=B + 2))
    q, k, v = t(B, H, 128), t(B, H, 64, 128), t(B, H, 64, 128)
    seq, o = t(B, dtype=torch.int32), t(B, H, 128)
    raises_device(mla.mla_mha_decode, q, k, v, seq, 64, o)
    raises_shape(mla.mla_mha_decode, q, k, t(B, H, 32, 128), seq, 64, o)
    raises_shape(mla.mla_mha_decode, q, k, v, seq, 64, t(B, H - 1, 128))
    with pytest.raises(ValueError, match="max_seq_len"):
        mla.mla_mha_decode(q, k, v, seq, 65, o)


def test_meta_tensors_are_not_device_buffers():
    m = torch.empty(B, H, 576, dtype=torch.bfloat16, device="meta")
    raises_device(mla.mla_decode, GEO, m, good_cache(), S, t(B, S, H, 512),
                  t(B, S, H, dtype=torch.float32))

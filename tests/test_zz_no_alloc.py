"""The no-allocation decode + tail (mla_decode_combine_up_proj_noalloc,
partials in the library's static device scratch) against the entry points it
composes (mla_decode into caller buffers, then mla_combine_up_proj): the same
kernels on the same inputs, so o, u and lse agree bit for bit.  Two calls in a
row, the second smaller, so the second reads nothing the first left in the
scratch; then a request beyond the scratch is refused on the host."""

import sys

import numpy as np
import pytest
import torch

import mla_latent_kv_15_amd as mla
import synth
from tests.device_inputs import DeviceInputs

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def _case(name, lens, S, seed):
    wl = synth.workload(name).with_(batch=len(lens), seq_len=None, num_splits=S, seed=seed)
    dev = DeviceInputs(synth.make_inputs(wl, lengths=lens))
    B, H = wl.batch, wl.heads
    q_abs = torch.empty(B, H, 576, dtype=torch.bfloat16, device="cuda")
    mla.mla_absorb_q(dev.geo, dev.q_nope, dev.q_rope, dev.w_uk, q_abs)
    return wl, dev, q_abs


def _reference(wl, dev, q_abs, S):
    B, H = wl.batch, wl.heads
    up = torch.empty(B, S, H, 512, dtype=torch.bfloat16, device="cuda")
    lp = torch.empty(B, S, H, dtype=torch.float32, device="cuda")
    mla.mla_decode(dev.geo, q_abs, dev.cache, S, up, lp)
    o = torch.empty(B, H, wl.d_v, dtype=torch.bfloat16, device="cuda")
    u = torch.empty(B, H, 512, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, H, dtype=torch.float32, device="cuda")
    mla.mla_combine_up_proj(dev.geo, up, lp, dev.w_uv, o, u, lse)
    return o, u, lse


def _noalloc(wl, dev, q_abs, S):
    B, H = wl.batch, wl.heads
    o = torch.full((B, H, wl.d_v), float("nan"), dtype=torch.bfloat16, device="cuda")
    u = torch.full((B, H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device="cuda")
    mla.mla_decode_combine_up_proj_noalloc(dev.geo, q_abs, dev.cache, S, dev.w_uv, o, u, lse)
    return o, u, lse


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("name", ["dsv2_b32_l2k", "paged_b64_ragged", "fp8_b1_l128k"])
def test_noalloc_matches_decode_then_fused_tail(name):
    # first call: 9 sequences (one empty, ragged), 6 splits; second call:
    # 3 shorter sequences, 2 splits -- fewer scratch rows than the first left
    calls = [([300, 0, 64, 1, 2047, 97, 33, 512, 8], 6, 0x51),
             ([45, 130, 7], 2, 0x52)]
    for lens, S, seed in calls:
        wl, dev, q_abs = _case(name, lens, S, synth.workloads.BASE_SEED + seed)
        _log(f"noalloc {name}: B={len(lens)} S={S}")
        got = _noalloc(wl, dev, q_abs, S)
        want = _reference(wl, dev, q_abs, S)
        torch.cuda.synchronize()
        for g, w, what in zip(got, want, ("o", "u", "lse")):
            assert torch.equal(_bits(g), _bits(w)), f"{name} B={len(lens)}: {what} differs"
        for b in (i for i, n in enumerate(lens) if n == 0):  # empty sequences
            assert torch.isneginf(got[2][b]).all() and (got[0][b].float() == 0).all()


def test_noalloc_largest_request_and_refusal():
    """The paged workload at full size sits exactly at the limit (64 x 8 x 128
    = 65536 rows) and matches; one more split is refused before any launch."""
    wl = synth.workload("paged_b64_ragged")
    dev = DeviceInputs(synth.make_inputs(wl))
    q_abs = torch.empty(wl.batch, wl.heads, 576, dtype=torch.bfloat16, device="cuda")
    mla.mla_absorb_q(dev.geo, dev.q_nope, dev.q_rope, dev.w_uk, q_abs)
    _log("noalloc paged full size, S=8")
    got = _noalloc(wl, dev, q_abs, 8)
    want = _reference(wl, dev, q_abs, 8)
    torch.cuda.synchronize()
    for g, w in zip(got, want):
        assert torch.equal(_bits(g), _bits(w))
    with pytest.raises(mla.MLAError) as e:
        _noalloc(wl, dev, q_abs, 9)
    assert e.value.status == 7  # MLA_E_SCRATCH
    assert np.isfinite(got[0].float().cpu().numpy()).all()

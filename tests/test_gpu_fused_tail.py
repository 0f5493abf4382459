"""GPU: mla_combine_up_proj (split merge + W_UV in one launch) against the
two-call path mla_combine -> mla_up_proj and against the CPU oracle.

The fused kernel rounds the merged u to bf16 exactly like mla_combine with a
bf16 u; the log-sum-exp normaliser is summed in a different lane order, so u
may differ in the last bf16 place.  o is compared with the oracle at the bf16
tolerance and with the two-call result at 1e-2 of max|o|."""

import numpy as np
import pytest
import torch

import mla_latent_kv_15_amd as mla
import synth
from tests.mla_cases import TOL, DeviceInputs, check_against_oracle, run_step

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")


def _log(msg):
    print(msg, flush=True)


def _two_call(dev, step, out_dtype):
    """merge + W_UV through the separate entry points, from step's partials"""
    g = step.geo
    B = step.B
    u = torch.empty(B, g.heads, g.d_latent, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, g.heads, dtype=torch.float32, device="cuda")
    o = torch.empty(B, g.heads, g.d_v, dtype=out_dtype, device="cuda")
    mla.mla_combine(g, step.u_part, step.lse_part, u, lse)
    mla.mla_up_proj(g, u, dev.w_uv, o)
    torch.cuda.synchronize()
    return u, lse, o


CASES = [  # (batch, lengths or uniform L, splits, partial dtype, output dtype)
    (7, [0, 1, 31, 300, 1000, 65, 2048], 4, torch.bfloat16, torch.bfloat16),
    (33, 777, 3, torch.bfloat16, torch.float32),
    (16, 1500, 1, torch.bfloat16, torch.bfloat16),
    (5, 4096, 64, torch.float32, torch.bfloat16),
    (20, 2000, 17, torch.float32, torch.float32),
    # one sequence: two workgroups per head, each with half of the value rows
    (1, 5000, 37, torch.bfloat16, torch.bfloat16),
    (1, 3000, 256, torch.bfloat16, torch.float32),
    (1, 700, 5, torch.float32, torch.bfloat16),
    # many splits: fewer sequences per workgroup than the grid alone would need
    (8, 9000, 256, torch.bfloat16, torch.bfloat16),
    (33, 500, 64, torch.bfloat16, torch.float32),
    # more workgroups than CUs: two per CU, W_UV rows loaded after the merge
    (70, 1200, 5, torch.float32, torch.bfloat16),
    (64, 2000, 40, torch.bfloat16, torch.float32),
]


@pytest.mark.parametrize("B,lens,S,part,out", CASES)
def test_fused_tail_matches_two_calls_and_oracle(B, lens, S, part, out):
    uniform = isinstance(lens, int)
    wl = synth.workload("dsv2_b32_l2k").with_(batch=B, seq_len=lens if uniform else None,
                                             seed=synth.workloads.BASE_SEED + 300 + B + S)
    dev = DeviceInputs(synth.make_inputs(wl, lengths=None if uniform else lens))
    step = run_step(dev, S, part_dtype=part, out_dtype=out)  # partials (and the default tail)
    u2, lse2, o2 = _two_call(dev, step, out)
    u = torch.empty_like(u2)
    lse = torch.empty_like(lse2)
    o = torch.empty_like(o2)
    mla.mla_combine_up_proj(step.geo, step.u_part, step.lse_part, dev.w_uv, o, u, lse)
    o_only = torch.empty_like(o2)
    mla.mla_combine_up_proj(step.geo, step.u_part, step.lse_part, dev.w_uv, o_only)
    torch.cuda.synchronize()
    # u within one bf16 place of mla_combine's: the two sum the splits in
    # different orders, so a rounding may flip (across a power of two that
    # place is the one of the larger value), plus the fp32 reordering error,
    # which is absolute on the scale of the summands (an element near zero
    # after cancellation has no relative bound); lse equal up to fp32 rounding
    du = (u.float() - u2.float()).abs()
    row = u2.float().abs().amax(dim=-1, keepdim=True)
    bound = 2.0 ** -7 * torch.maximum(u.float().abs(), u2.float().abs()) + 2.0 ** -14 * row
    assert torch.all(du <= bound + 1e-30), du.max().item()
    fin = torch.isfinite(lse2)
    assert torch.equal(fin, torch.isfinite(lse))
    assert torch.allclose(lse[fin], lse2[fin], rtol=0, atol=1e-5)
    assert torch.equal(o.view(torch.int16) if out == torch.bfloat16 else o,
                       o_only.view(torch.int16) if out == torch.bfloat16 else o_only)
    scale = o2.float().abs().max().item()
    err = (o.float() - o2.float()).abs().max().item()
    assert err <= 1e-2 * max(scale, 1e-30), (err, scale)
    # and the fused result against the oracle, through the step object
    step.u.copy_(u.to(step.u.dtype))
    step.lse.copy_(lse)
    step.o.copy_(o)
    pairs = [(b, h) for b in sorted({0, B // 2, B - 1}) for h in (0, 77, 127)]
    e = check_against_oracle(dev, step, pairs, TOL["bf16"])
    _log(f"fused tail B={B} S={S}: |o - two-call| {err:.2e} of {scale:.2e}; oracle {e}")

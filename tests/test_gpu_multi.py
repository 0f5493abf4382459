"""GPU: multi-token decode (mla_decode_multi, q_len query tokens per sequence
attending causally to the cache) through the C ABI, finished by
mla_combine_up_proj over B*q_len rows, against the oracle run once per query
token with the attended range cut at that token."""

import numpy as np
import pytest
import torch

import mla_latent_kv_15_amd as mla
import oracle
import synth
from synth.encode import f32_to_bf16_bits
from tests.mla_cases import TOL, DeviceInputs, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")


def _log(msg):
    print(msg, flush=True)


def _bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


AUTO, H64 = mla.KERNEL_AUTO, mla.KERNEL_H64
CASES = [("dsv2_b32_l2k", 2, 3, AUTO), ("dsv2_b32_l2k", 4, 1, AUTO), ("paged_b64_ragged", 3, 4, AUTO),
         ("fp8_b1_l128k", 4, 3, AUTO), ("dsv2_b32_l2k", 4, 3, H64), ("paged_b64_ragged", 2, 4, H64),
         ("dsv2_b32_l2k", 16, 2, AUTO)]  # the largest q_len the ABI takes


@pytest.mark.parametrize("name,ql,S,kernel", CASES)
def test_multi_token_decode_matches_oracle(name, ql, S, kernel):
    lens = np.array([300, 2, 64, 97, 1], np.int32)  # lengths below q_len: early queries see nothing
    B = len(lens)
    wl = synth.workload(name).with_(batch=B, seq_len=None, num_splits=S,
                                    seed=synth.workloads.BASE_SEED + 150 + ql)
    inp = synth.make_inputs(wl, lengths=lens.tolist())
    dev = DeviceInputs(inp)
    H = wl.heads
    r = np.random.default_rng(150 + ql)
    qn = f32_to_bf16_bits(r.standard_normal((B, ql, H, wl.d_nope)).astype(np.float32))
    qr = f32_to_bf16_bits(r.standard_normal((B, ql, H, wl.d_rope)).astype(np.float32))
    q_abs = torch.empty(B, ql, H, 576, dtype=torch.bfloat16, device="cuda")
    mla.mla_absorb_q(dev.geo, _bf16_dev(qn).view(B * ql, H, -1), _bf16_dev(qr).view(B * ql, H, -1),
                     dev.w_uk, q_abs.view(B * ql, H, 576))
    u_part = torch.empty(B, ql, S, H, 512, dtype=torch.bfloat16, device="cuda")
    lse_part = torch.empty(B, ql, S, H, dtype=torch.float32, device="cuda")
    _log(f"multi-token {name} q_len={ql} S={S} kernel={kernel}")
    if kernel == AUTO:
        mla.mla_decode_multi(dev.geo, q_abs, dev.cache, S, u_part, lse_part)
    else:
        mla.mla_decode_ex(dev.geo, q_abs, dev.cache, S, u_part, lse_part, kernel=kernel)
    o = torch.empty(B * ql, H, wl.d_v, dtype=torch.bfloat16, device="cuda")
    u = torch.empty(B * ql, H, 512, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B * ql, H, dtype=torch.float32, device="cuda")
    mla.mla_combine_up_proj(dev.geo, u_part.view(B * ql, S, H, 512), lse_part.view(B * ql, S, H),
                            dev.w_uv, o, u, lse)
    torch.cuda.synchronize()
    o, u, lse = (t.float().cpu().numpy() for t in (o, u, lse))
    tol = TOL["fp8" if wl.cache_dtype == "fp8" else "bf16"]
    pairs = [(b, h) for b in range(B) for h in (0, 77, 127)]
    for j in range(ql):
        t_end = np.maximum(lens - (ql - 1 - j), 0).astype(np.int32)
        o_ref, lse_ref, u_ref = oracle.decode(
            qn[:, j], qr[:, j], "bf16", inp.w_uk, inp.w_uv, "bf16", inp.rows, wl.cache_dtype,
            inp.seq_lens, row_scale=inp.row_scale, page_size=wl.page_size,
            seq_stride=inp.seq_stride, block_table=inp.block_table, sel=pairs, t_end=t_end,
            want_u=True)
        rows = [b * ql + j for b, _ in pairs]
        hs = [h for _, h in pairs]
        e_o = rel_err(o[rows, hs], o_ref)
        e_u = rel_err(u[rows, hs], u_ref)
        lg = lse[rows, hs]
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isfinite(lg), fin)
        e_l = float(np.abs(lg[fin] - lse_ref[fin]).max()) if fin.any() else 0.0
        _log(f"  j={j}: err o/u/lse = {e_o:.2e} {e_u:.2e} {e_l:.2e}")
        assert e_o <= tol and e_u <= tol and e_l <= tol

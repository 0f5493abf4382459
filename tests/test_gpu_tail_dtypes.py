"""GPU: the tail of the step for every provided dtype combination, through the
C ABI, against the oracle on the same stored values: mla_up_proj (o = W_UV u)
and mla_combine (log-sum-exp merge of split partials, empty ranges included)."""

import numpy as np
import pytest
import torch

import mla_latent_kv_15_amd as mla
import oracle
from synth.encode import bf16_bits_to_f32, f32_to_bf16_bits

pytestmark = pytest.mark.gpu

F32, BF16 = "f32", "bf16"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")


def _log(msg):
    print(msg, flush=True)


def _stored(x, dt):
    """The values the GPU reads: float32, or bf16 bits (returned as float64)."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x)).astype(np.float64) if dt == BF16 else x.astype(np.float64)


def _dev(x, dt):
    if dt == BF16:
        return torch.from_numpy(f32_to_bf16_bits(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()


def _empty(shape, dt):
    return torch.empty(shape, dtype=torch.float32 if dt == F32 else torch.bfloat16, device="cuda")


# tolerance relative to the largest reference value: one bf16 rounding of the
# output, or fp32 accumulation
def _tol(dt):
    return 2.0 ** -8 if dt == BF16 else 1e-5


UP_DTYPES = [(F32, F32, F32), (F32, BF16, F32), (F32, BF16, BF16), (BF16, BF16, BF16),
             (BF16, BF16, F32), (F32, F32, BF16)]


@pytest.mark.parametrize("u_dt,w_dt,o_dt", UP_DTYPES)
def test_up_proj_dtypes_match_oracle(u_dt, w_dt, o_dt):
    B, H = 37, 128  # more than one 32-sequence tile of the matrix-core kernel
    r = np.random.default_rng(141)
    u = (r.standard_normal((B, H, 512)) * 0.1).astype(np.float32)
    w = (r.standard_normal((H, 128, 512)) / np.sqrt(512)).astype(np.float32)
    o = _empty((B, H, 128), o_dt)
    _log(f"up_proj u={u_dt} w={w_dt} o={o_dt}")
    mla.mla_up_proj(mla.Geometry(heads=H), _dev(u, u_dt), _dev(w, w_dt), o)
    torch.cuda.synchronize()
    w_bits = f32_to_bf16_bits(w) if w_dt == BF16 else w
    want = oracle.up_proj(_stored(u, u_dt), w_bits, w_dt)
    err = np.abs(o.float().cpu().numpy() - want).max() / np.abs(want).max()
    _log(f"  max rel err {err:.2e}")
    assert err <= _tol(o_dt)


COMBINE_DTYPES = [(F32, F32), (F32, BF16), (BF16, F32), (BF16, BF16)]


@pytest.mark.parametrize("part_dt,u_dt", COMBINE_DTYPES)
def test_combine_dtypes_match_oracle(part_dt, u_dt):
    B, S, H = 37, 5, 128
    r = np.random.default_rng(142)
    up = r.standard_normal((B, S, H, 512)).astype(np.float32)
    lse = (r.standard_normal((B, S, H)) * 3.0).astype(np.float32)
    lse[3, 2:] = -np.inf  # trailing empty ranges (their partials are zero)
    up[3, 2:] = 0.0
    lse[5] = -np.inf  # an empty sequence
    up[5] = 0.0
    u = _empty((B, H, 512), u_dt)
    lse_out = torch.empty(B, H, dtype=torch.float32, device="cuda")
    _log(f"combine parts={part_dt} u={u_dt}")
    mla.mla_combine(mla.Geometry(heads=H), _dev(up, part_dt), torch.from_numpy(lse).cuda(), u,
                    lse_out)
    torch.cuda.synchronize()
    u_ref, lse_ref = oracle.combine(_stored(up, part_dt), lse.astype(np.float64))
    got = u.float().cpu().numpy()
    assert np.all(got[5] == 0.0) and np.all(np.isneginf(lse_out[5].cpu().numpy()))
    err = np.abs(got - u_ref).max() / np.abs(u_ref).max()
    fin = np.isfinite(lse_ref)
    e_l = np.abs(lse_out.cpu().numpy()[fin] - lse_ref[fin]).max()
    _log(f"  max rel err u {err:.2e}, lse {e_l:.2e}")
    assert err <= _tol(u_dt) and e_l <= 1e-5

"""GPU: mla_absorb_q_rope through the C ABI.  The rotated positional part
against the oracle's RoPE, the latent part bit for bit against mla_absorb_q,
and a decode step with the rotated query against the oracle run on the
oracle-rotated query."""

import numpy as np
import pytest
import torch

import mla_latent_kv_15_amd as mla
import oracle
import synth
from tests.mla_cases import TOL, DeviceInputs, rel_err, run_step

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")


def _log(msg):
    print(msg, flush=True)


def _bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 \
        else t.cpu().numpy()


# (workload giving the q/W dtypes, q_abs dtype): the bf16 matrix-core kernel
# with bf16 and fp32 output, and the fp32 VALU kernel
CASES = [("dsv2_b32_l2k", torch.bfloat16), ("dsv2_b32_l2k", torch.float32),
         ("tiny_f32", torch.float32)]


@pytest.mark.parametrize("name,qa_dt", CASES)
@pytest.mark.parametrize("B", [5, 37])
def test_absorb_rope_matches_oracle(name, qa_dt, B):
    wl = synth.workload(name).with_(batch=B, seq_len=64, seed=synth.workloads.BASE_SEED + 130)
    inp = synth.make_inputs(wl)
    dev = DeviceInputs(inp)
    pos = np.random.default_rng(B).integers(0, 131072, size=B).astype(np.int32)
    pos[:3] = [0, 131071, -300]
    q_abs = torch.empty(B, wl.heads, 576, dtype=qa_dt, device="cuda")
    q_ref = torch.empty_like(q_abs)
    _log(f"absorb rope {name} q_abs={qa_dt} B={B}")
    mla.mla_absorb_q_rope(dev.geo, dev.q_nope, dev.q_rope, dev.w_uk, torch.from_numpy(pos).cuda(),
                          q_abs)
    mla.mla_absorb_q(dev.geo, dev.q_nope, dev.q_rope, dev.w_uk, q_ref)
    torch.cuda.synchronize()
    got, plain = _bits(q_abs), _bits(q_ref)
    # the latent part is mla_absorb_q's, bit for bit; position 0 leaves q_R as it is
    assert np.array_equal(got[..., :512], plain[..., :512])
    assert np.array_equal(got[0, :, 512:], plain[0, :, 512:])
    want = oracle.rope(inp.q_rope, wl.act_dtype, pos)
    g = q_abs[..., 512:].float().cpu().numpy().astype(np.float64)
    scale = np.abs(want).max(axis=-1, keepdims=True)
    # bf16 output: one rounding (2^-9 relative) of a value up to the row's
    # maximum; fp32 output: binary32 sincos and products
    tol = 2.0 ** -8 if qa_dt == torch.bfloat16 else 2e-6
    err = np.abs(g - want) / scale
    _log(f"  max rel err {err.max():.2e}")
    assert err.max() <= tol


@pytest.mark.parametrize("name", ["dsv2_b32_l2k", "fp8_b1_l128k"])
def test_decode_with_rotated_query(name):
    lens = [300, 1, 64, 97]
    wl = synth.workload(name).with_(batch=len(lens), seq_len=None, num_splits=3,
                                    seed=synth.workloads.BASE_SEED + 131)
    inp = synth.make_inputs(wl, lengths=lens)
    dev = DeviceInputs(inp)
    pos = np.array([299, 5000, 64, 131071], np.int32)
    step = mla.DecodeStep(dev.geo, wl.batch, wl.num_splits, act_dtype=torch.bfloat16,
                          part_dtype=torch.bfloat16, out_dtype=torch.bfloat16)
    _log(f"decode with rotated query: {name}")
    mla.mla_absorb_q_rope(dev.geo, dev.q_nope, dev.q_rope, dev.w_uk, torch.from_numpy(pos).cuda(),
                          step.q_abs)
    mla.mla_decode(dev.geo, step.q_abs, dev.cache, wl.num_splits, step.u_part, step.lse_part)
    mla.mla_combine_up_proj(dev.geo, step.u_part, step.lse_part, dev.w_uv, step.o)
    torch.cuda.synchronize()
    q_nope64 = oracle.decode_array(inp.q_nope, wl.act_dtype)
    q_rope64 = oracle.rope(inp.q_rope, wl.act_dtype, pos)
    pairs = [(b, h) for b in range(len(lens)) for h in (0, 77, 127)]
    o_ref, _, _ = oracle.decode(q_nope64, q_rope64, "f64", inp.w_uk, inp.w_uv, wl.act_dtype,
                                inp.rows, wl.cache_dtype, inp.seq_lens, row_scale=inp.row_scale,
                                page_size=wl.page_size, seq_stride=inp.seq_stride,
                                block_table=inp.block_table, sel=pairs)
    o = step.o.float().cpu().numpy()
    e = rel_err(np.stack([o[b, h] for b, h in pairs]), o_ref)
    _log(f"  o err {e:.2e}")
    assert e <= TOL["fp8" if wl.cache_dtype == "fp8" else "bf16"]


F32, BF16 = "f32", "bf16"
ABSORB_DTYPES = [(F32, F32, F32), (F32, F32, BF16), (BF16, BF16, BF16), (BF16, BF16, F32),
                 (F32, BF16, BF16), (BF16, F32, BF16)]


@pytest.mark.parametrize("q_dt,w_dt,out_dt", ABSORB_DTYPES)
def test_absorb_dtypes_match_oracle(q_dt, w_dt, out_dt):
    """mla_absorb_q for every provided (query, weight, output) dtype triple
    against the oracle's absorbed query (float64 over the same stored bits):
    the matrix-core kernel for bf16/bf16 and the VALU kernel for the rest, 37
    sequences (more than one tile of 32)."""
    from synth.encode import f32_to_bf16_bits
    B, H, dn = 37, 128, 128
    r = np.random.default_rng(140)
    qn = r.standard_normal((B, H, dn)).astype(np.float32)
    qr = r.standard_normal((B, H, 64)).astype(np.float32)
    wk = (r.standard_normal((H, dn, 512)) / np.sqrt(512)).astype(np.float32)

    def stored(x, dt):  # the bits both sides read
        return f32_to_bf16_bits(x) if dt == BF16 else x

    def dev(x, dt):
        if dt == BF16:
            return torch.from_numpy(stored(x, dt).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(x).cuda()

    geo = mla.Geometry(heads=H)
    q_abs = torch.empty(B, H, 576, dtype=torch.float32 if out_dt == F32 else torch.bfloat16,
                        device="cuda")
    _log(f"absorb q={q_dt} w={w_dt} out={out_dt}")
    mla.mla_absorb_q(geo, dev(qn, q_dt), dev(qr, q_dt), dev(wk, w_dt), q_abs)
    torch.cuda.synchronize()
    want = oracle.absorb_q(stored(qn, q_dt), stored(qr, q_dt), q_dt, stored(wk, w_dt), w_dt)
    got = q_abs.float().cpu().numpy().astype(np.float64)
    scale = np.abs(want).max(axis=-1, keepdims=True)
    # bf16 output: one rounding; fp32 output: fp32 accumulation over d_nope products
    tol = 2.0 ** -8 if out_dt == BF16 else 1e-5
    err = (np.abs(got - want) / scale).max()
    _log(f"  max rel err {err:.2e}")
    assert err <= tol


@pytest.mark.parametrize("dn", [64, 192, 256])
@pytest.mark.parametrize("out_dt", [BF16, F32])
def test_absorb_other_head_dims_match_oracle(dn, out_dt):
    """The matrix-core absorb at d_nope other than 128: 64 takes the path that
    stages query rows and the output tile in LDS, 192 and 256 the path that
    keeps the query operands in registers and stores from the accumulators
    (37 sequences: a full tile of 32 and a ragged one)."""
    from synth.encode import f32_to_bf16_bits, bf16_bits_to_f32
    B, H = 37, 16
    r = np.random.default_rng(143 + dn)
    qn = f32_to_bf16_bits(r.standard_normal((B, H, dn)).astype(np.float32))
    qr = f32_to_bf16_bits(r.standard_normal((B, H, 64)).astype(np.float32))
    wk = f32_to_bf16_bits((r.standard_normal((H, dn, 512)) / np.sqrt(512)).astype(np.float32))

    def dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()

    geo = mla.Geometry(heads=H, d_nope=dn)
    q_abs = torch.empty(B, H, 576, dtype=torch.float32 if out_dt == F32 else torch.bfloat16,
                        device="cuda")
    _log(f"absorb d_nope={dn} out={out_dt}")
    mla.mla_absorb_q(geo, dev(qn), dev(qr), dev(wk), q_abs)
    torch.cuda.synchronize()
    want = oracle.absorb_q(qn, qr, BF16, wk, BF16)
    got = q_abs.float().cpu().numpy().astype(np.float64)
    assert np.array_equal(got[..., 512:], bf16_bits_to_f32(qr).astype(np.float64))
    scale = np.abs(want).max(axis=-1, keepdims=True)
    tol = 2.0 ** -8 if out_dt == BF16 else 1e-5
    err = (np.abs(got - want) / scale).max()
    _log(f"  max rel err {err:.2e}")
    assert err <= tol

"""GPU: the ring cache through the C ABI against the oracle.  Appends that wrap
around the ring (bf16 and fp8 rows, bit for bit), a decode step over rings
that have wrapped (sequences longer than the capacity attend their last C
tokens), and growing / shrinking a ring (bit for bit)."""

import dataclasses
import sys

import numpy as np
import pytest
import torch

import mla_latent_kv_15_amd as mla
import oracle
import synth
from synth.encode import f32_to_bf16_bits
from tests.device_inputs import DeviceInputs, bits_to_tensor
from tests.mla_cases import TOL, check_against_oracle, run_step

pytestmark = pytest.mark.gpu

DL, DR, W = 512, 64, 576
NP = {"bf16": np.uint16, "fp8": np.uint8}


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def _dev_bits(t, dt):
    return t.cpu().view(torch.int16).numpy().view(np.uint16) if dt == "bf16" else t.cpu().numpy()


@pytest.mark.parametrize("cache_dt", ["bf16", "fp8"])
def test_ring_append_wraps_like_the_oracle(cache_dt):
    """Positions past the capacity overwrite row t % C of the sequence's ring;
    negative positions are skipped."""
    B, C = 6, 40
    r = np.random.default_rng(71)
    rows = r.integers(0, 2 ** (16 if cache_dt == "bf16" else 8), (B * C, W)).astype(NP[cache_dt])
    if cache_dt == "fp8":
        rows[(rows & 0x7F) == 0x7F] = 0  # no NaN codes in untouched rows
    scale = r.standard_normal(B * C).astype(np.float32) if cache_dt == "fp8" else None
    pos = np.array([0, 39, 40, 41, 1000, -1], np.int32)
    src = f32_to_bf16_bits(r.standard_normal((B, W)).astype(np.float32))
    want_rows, want_scale = rows.copy(), None if scale is None else scale.copy()
    oracle.cache_append(src[:, :DL], src[:, DL:], "bf16", pos, want_rows, cache_dt,
                        row_scale=want_scale, seq_stride=C, ring=True)
    d_rows = bits_to_tensor(rows, cache_dt)
    d_scale = None if scale is None else torch.from_numpy(scale.copy()).cuda()
    cache = mla.Cache(rows=d_rows, seq_lens=torch.zeros(B, dtype=torch.int32, device="cuda"),
                      max_seq_len=0, row_scale=d_scale, seq_stride=C, ring=True)
    _log(f"ring append {cache_dt}")
    mla.mla_cache_append(mla.Geometry(heads=128), bits_to_tensor(src[:, :DL], "bf16"),
                         bits_to_tensor(src[:, DL:], "bf16"), torch.from_numpy(pos).cuda(), cache)
    torch.cuda.synchronize()
    assert np.array_equal(_dev_bits(d_rows, cache_dt), want_rows)
    if scale is not None:
        assert np.array_equal(d_scale.cpu().numpy().view(np.uint32), want_scale.view(np.uint32))


@pytest.mark.parametrize("name,S", [("dsv2_b32_l2k", 3), ("fp8_b1_l128k", 2), ("tiny_f32", 2)])
def test_decode_over_wrapped_rings(name, S):
    """Rings of capacity 200: sequences of 1000 and 201 tokens have wrapped and
    attend their last 200 tokens; 200, 57 and 0 tokens fit.  The ring holds
    min(L, C) written rows; the rest are NaN and must stay unread."""
    C = 200
    lens = [1000, 201, 200, 57, 0] if name != "tiny_f32" else [1000, 57]
    wl = synth.workload(name).with_(batch=len(lens), seq_len=None, num_splits=S,
                                    seed=synth.workloads.BASE_SEED + 160)
    inp = synth.make_inputs(wl, lengths=[min(n, C) for n in lens], seq_stride=C)
    inp = dataclasses.replace(inp, seq_lens=np.asarray(lens, np.int32), max_seq_len=max(lens))
    dev = DeviceInputs(inp)
    dev.cache.ring = True
    _log(f"ring decode {name} S={S}")
    step = run_step(dev, S)
    pairs = [(b, h) for b in range(len(lens)) for h in sorted({0, wl.heads // 2, wl.heads - 1})]
    o_ref, lse_ref, u_ref = oracle.decode_inputs(inp, sel=pairs, want_u=True, ring=True)
    kind = {"bf16": "bf16", "fp8": "fp8", "f32": "f32"}[wl.cache_dtype]
    e = check_against_oracle_ring(step, pairs, o_ref, lse_ref, u_ref, TOL[kind])
    _log(f"  err o/u/lse = {e}")


def check_against_oracle_ring(step, pairs, o_ref, lse_ref, u_ref, tol):
    o = step.o.float().cpu().numpy()
    u = step.u.float().cpu().numpy()
    lse = step.lse.float().cpu().numpy()
    o_got = np.stack([o[b, h] for b, h in pairs])
    u_got = np.stack([u[b, h] for b, h in pairs])
    l_got = np.array([lse[b, h] for b, h in pairs])
    assert np.all(np.isfinite(o_got)) and np.all(np.isfinite(u_got))
    e_o = np.abs(o_got - o_ref).max() / np.abs(o_ref).max()
    e_u = np.abs(u_got - u_ref).max() / np.abs(u_ref).max()
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(l_got), fin)
    e_l = np.abs(l_got[fin] - lse_ref[fin]).max()
    assert e_o <= tol and e_u <= tol and e_l <= tol, (e_o, e_u, e_l)
    return e_o, e_u, e_l


@pytest.mark.parametrize("cache_dt,C,C2", [("bf16", 96, 160), ("bf16", 96, 40), ("fp8", 64, 128)])
def test_ring_grow_matches_the_oracle(cache_dt, C, C2):
    lens = [500, 96, 30, 0, 64]
    B = len(lens)
    r = np.random.default_rng(C + C2)
    rows = r.integers(0, 2 ** (16 if cache_dt == "bf16" else 8), (B * C, W)).astype(NP[cache_dt])
    scale = r.standard_normal(B * C).astype(np.float32) if cache_dt == "fp8" else None
    want, want_scale = oracle.ring_grow(lens, rows, C, C2, src_scale=scale)
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
    src = mla.Cache(rows=bits_to_tensor(rows, cache_dt), seq_lens=seq, max_seq_len=max(lens),
                    row_scale=None if scale is None else torch.from_numpy(scale).cuda(),
                    seq_stride=C, ring=True)
    d_rows = bits_to_tensor(np.zeros((B * C2, W), NP[cache_dt]), cache_dt)
    d_scale = None if scale is None else torch.zeros(B * C2, dtype=torch.float32, device="cuda")
    dst = mla.Cache(rows=d_rows, seq_lens=seq, max_seq_len=max(lens), row_scale=d_scale,
                    seq_stride=C2, ring=True)
    _log(f"ring grow {cache_dt} {C} -> {C2}")
    mla.mla_cache_ring_grow(mla.Geometry(heads=128), src, dst)
    torch.cuda.synchronize()
    assert np.array_equal(_dev_bits(d_rows, cache_dt), want)
    if scale is not None:
        assert np.array_equal(d_scale.cpu().numpy().view(np.uint32), want_scale.view(np.uint32))

"""GPU: the E4M3 absorbed query and the fp8 matrix-core decode through the C
ABI, against the oracle.

* mla_absorb_q with an E4M3 output: every code within half an E4M3 step of the
  oracle's float64 absorbed query, the factor = the row's largest magnitude /
  448 (one factor per (sequence, head), the fp8 cache rows' rule);
* mla_decode with an E4M3 query on an E4M3 cache: the same stored query codes
  and factors go to the kernel and to the oracle's absorbed-form attention, so
  the comparison isolates the kernel (its E4M3 probabilities and bf16
  partials) from the query's own rounding: contiguous, paged and ring caches,
  odd lengths (a pair of rows whose second row is past the end), a one-token
  sequence, empty sequences, 32 and 128 heads, several splits;
* the score-spike redo on this path.
* workgroups that take several consecutive split ranges and merge them
  (many splits and few sequences: 256 splits at 2 x 128 heads gives 4 ranges
  per workgroup, merged into one split), including groups past the end of a
  sequence, a group that straddles it, and a score-spike redo of a group.
The end-to-end step (absorb -> decode -> tail) at the full 128K sizes is in
test_gpu_parity.py (the "fp8 query" cases)."""

import dataclasses
import sys

import numpy as np
import pytest
import torch

import mla_latent_kv_15_amd as mla
import oracle
import synth
from synth.encode import quantize_rows_e4m3
from tests.device_inputs import DeviceInputs, bits_to_tensor
from tests.mla_cases import ranges_per_split

pytestmark = pytest.mark.gpu

TOL_FP8 = 6e-2


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    assert np.all(np.isfinite(a)), "non-finite GPU output"
    return float(np.abs(a - b).max() / np.abs(b).max())


@pytest.mark.parametrize("B,H", [(1, 128), (8, 128), (40, 32)])
def test_absorb_fp8_output(B, H):
    wl = synth.workload("fp8_b1_l128k").with_(batch=B, heads=H, seq_len=64,
                                              seed=synth.workloads.BASE_SEED + 400 + B)
    inp = synth.make_inputs(wl)
    dev = DeviceInputs(inp)
    codes = torch.zeros(B, H, 576, dtype=torch.uint8, device="cuda")
    scale = torch.zeros(B, H, dtype=torch.float32, device="cuda")
    _log(f"absorb fp8 B={B} H={H}")
    mla.mla_absorb_q(dev.geo, dev.q_nope, dev.q_rope, dev.w_uk, codes, scale)
    torch.cuda.synchronize()
    qa = oracle.absorb_q(inp.q_nope, inp.q_rope, "bf16", inp.w_uk, "bf16")
    sc = scale.cpu().numpy()
    sc_ref = np.abs(qa).max(axis=-1) / 448.0
    assert np.abs(sc / sc_ref - 1).max() <= 1e-5
    dq = oracle.decode_array(codes.cpu().numpy(), "fp8") * sc.astype(np.float64)[..., None]
    # half an E4M3 step of the value (2^-4 relative; 2^-10 of the factor in
    # the subnormal range), plus the fp32 accumulation's own error
    step = np.maximum(np.abs(qa) * 2.0 ** -4, sc.astype(np.float64)[..., None] * 2.0 ** -10)
    err = np.abs(dq - qa) - step * (1 + 1e-3) - np.abs(qa) * 1e-5
    assert err.max() <= 0.0, float(err.max())


def _query(B, H, seed):
    """synthetic absorbed query rows (latent part N(0, 1/4) like W_UK^T q_C with
    W_UK ~ N(0, 1/512), RoPE part N(0, 1)) as E4M3 codes + factors"""
    r = np.random.default_rng(seed)
    q = r.standard_normal((B * H, 576)).astype(np.float32)
    q[:, :512] *= 0.5
    codes, scale = quantize_rows_e4m3(q)
    return codes.reshape(B, H, 576), scale.reshape(B, H)


def _decode(dev, codes, scale, S, part=torch.bfloat16):
    B, H = codes.shape[:2]
    u_part = torch.full((B, S, H, 512), float("nan"), dtype=part, device="cuda")
    lse_part = torch.full((B, S, H), float("nan"), dtype=torch.float32, device="cuda")
    q = bits_to_tensor(codes, "fp8")
    qs = torch.from_numpy(np.ascontiguousarray(scale)).cuda()
    mla.mla_decode(dev.geo, q, dev.cache, S, u_part, lse_part, q_abs_scale=qs)
    u = torch.empty(B, H, 512, dtype=torch.float32, device="cuda")
    lse = torch.empty(B, H, dtype=torch.float32, device="cuda")
    mla.mla_combine(dev.geo, u_part, lse_part, u, lse)
    torch.cuda.synchronize()
    return u.cpu().numpy(), lse.cpu().numpy(), u_part, lse_part


def _check(inp, codes, scale, u, lse, pairs, ring=False):
    wl = inp.wl
    u_ref, l_ref, _ = oracle.absorbed_decode(
        codes, "fp8", inp.rows, "fp8", inp.seq_lens, q_scale=scale, row_scale=inp.row_scale,
        page_size=wl.page_size, seq_stride=inp.seq_stride, block_table=inp.block_table,
        sel=pairs, ring=ring)
    u_got = np.stack([u[b, h] for b, h in pairs])
    l_got = np.array([lse[b, h] for b, h in pairs])
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isfinite(l_got), fin)
    assert np.all(u_got[~fin] == 0.0)
    e_u = _rel(u_got[fin], u_ref[fin])
    e_l = float(np.abs(l_got[fin] - l_ref[fin]).max())
    return e_u, e_l


CASES = [
    # name, lens, heads, S, page size
    ("contig", [300, 64, 1, 0, 129], 128, 2, 0),
    ("paged", [1000, 65, 63, 2], 128, 4, 64),
    ("h32", [77, 500, 190], 32, 3, 0),
    ("one_split", [450, 33], 128, 1, 0),
]


@pytest.mark.parametrize("name,lens,H,S,ps", CASES, ids=[c[0] for c in CASES])
def test_fp8_query_decode_matches_the_oracle(name, lens, H, S, ps):
    wl = synth.workload("fp8_b1_l128k").with_(batch=len(lens), heads=H, seq_len=None,
                                              page_size=ps, seed=synth.workloads.BASE_SEED + 410)
    inp = synth.make_inputs(wl, lengths=lens)
    dev = DeviceInputs(inp)
    codes, scale = _query(len(lens), H, 411)
    _log(f"fp8 query decode {name} S={S}")
    u, lse, _, _ = _decode(dev, codes, scale, S)
    pairs = [(b, h) for b in range(len(lens)) for h in sorted({0, 31, H // 2, H - 1})]
    e_u, e_l = _check(inp, codes, scale, u, lse, pairs)
    _log(f"  err u {e_u:.2e} lse {e_l:.2e}")
    assert e_u <= TOL_FP8 and e_l <= TOL_FP8


def test_fp8_query_decode_over_wrapped_rings():
    C = 200
    lens = [1000, 201, 57, 0]
    wl = synth.workload("fp8_b1_l128k").with_(batch=len(lens), heads=128, seq_len=None,
                                              seed=synth.workloads.BASE_SEED + 412)
    inp = synth.make_inputs(wl, lengths=[min(n, C) for n in lens], seq_stride=C)
    inp = dataclasses.replace(inp, seq_lens=np.asarray(lens, np.int32), max_seq_len=max(lens))
    dev = DeviceInputs(inp)
    dev.cache.ring = True
    codes, scale = _query(len(lens), 128, 413)
    _log("fp8 query decode ring")
    u, lse, _, _ = _decode(dev, codes, scale, 2)
    pairs = [(b, h) for b in range(len(lens)) for h in (0, 77, 127)]
    e_u, e_l = _check(inp, codes, scale, u, lse, pairs, ring=True)
    _log(f"  err u {e_u:.2e} lse {e_l:.2e}")
    assert e_u <= TOL_FP8 and e_l <= TOL_FP8


def test_fp8_query_partials_every_split():
    """Each split range's partial (not only the merged result) against the
    oracle over that range, fp32 partials: ranges are whole 64-token tiles."""
    lens = [700, 129]
    S = 3
    wl = synth.workload("fp8_b1_l128k").with_(batch=2, heads=64, seq_len=None,
                                              seed=synth.workloads.BASE_SEED + 414)
    inp = synth.make_inputs(wl, lengths=lens)
    dev = DeviceInputs(inp)
    codes, scale = _query(2, 64, 415)
    _, _, u_part, lse_part = _decode(dev, codes, scale, S, part=torch.float32)
    up, lp = u_part.cpu().numpy(), lse_part.cpu().numpy()
    chunk = 64 * -(-max(lens) // (64 * S))
    for p in range(S):
        tb = [min(p * chunk, L) for L in lens]
        te = [min((p + 1) * chunk, L) for L in lens]
        pairs = [(b, h) for b in range(2) for h in (0, 40, 63)]
        u_ref, l_ref, _ = oracle.absorbed_decode(
            codes, "fp8", inp.rows, "fp8", inp.seq_lens, q_scale=scale, row_scale=inp.row_scale,
            seq_stride=inp.seq_stride, sel=pairs, t_begin=tb, t_end=te)
        for k, (b, h) in enumerate(pairs):
            if not np.isfinite(l_ref[k]):  # empty: lse = -inf, u not written
                assert np.isneginf(lp[b, p, h])
                continue
            assert abs(lp[b, p, h] - l_ref[k]) <= TOL_FP8, (p, b, h)
            assert _rel(up[b, p, h], u_ref[k]) <= TOL_FP8, (p, b, h)


def test_fp8_query_score_spike_recomputes_range():
    """One token whose score exceeds the first tile's maximum by far more than
    the reference slack: the range is computed again with the true maximum."""
    lens = [400]
    wl = synth.workload("fp8_b1_l128k").with_(batch=1, heads=32, seq_len=None,
                                              seed=synth.workloads.BASE_SEED + 416)
    inp = synth.make_inputs(wl, lengths=lens)
    codes, scale = _query(1, 32, 417)
    # token 300's row becomes the query direction of every head, scaled up
    rows = oracle.decode_array(inp.rows, "fp8") * inp.row_scale.astype(np.float64)[:, None]
    q = oracle.decode_array(codes, "fp8")[0] * scale[0].astype(np.float64)[:, None]
    spike = np.sign(q.mean(axis=0)) * 40.0
    r = inp.row_index(0, 300)
    c8, s8 = quantize_rows_e4m3(spike[None, :].astype(np.float32))
    new_rows = inp.rows.copy()
    new_rows[r] = c8[0]
    new_scale = inp.row_scale.copy()
    new_scale[r] = s8[0]
    inp = dataclasses.replace(inp, rows=new_rows, row_scale=new_scale)
    dev = DeviceInputs(inp)
    u, lse, _, _ = _decode(dev, codes, scale, 1)
    pairs = [(0, h) for h in (0, 13, 31)]
    u_ref, l_ref, _ = oracle.absorbed_decode(
        codes, "fp8", inp.rows, "fp8", inp.seq_lens, q_scale=scale, row_scale=inp.row_scale,
        seq_stride=inp.seq_stride, sel=pairs)
    s_first = (rows[:64] @ q.T).max() / np.sqrt(192.0) * np.log2(np.e)
    assert l_ref.min() * np.log2(np.e) > s_first + 64  # beyond the slack
    e_u = _rel(np.stack([u[b, h] for b, h in pairs]), u_ref)
    e_l = float(np.abs(np.array([lse[b, h] for b, h in pairs]) - l_ref).max())
    _log(f"spike: err u {e_u:.2e} lse {e_l:.2e}")
    assert e_u <= TOL_FP8 and e_l <= TOL_FP8


def test_fp8_query_multi_range_workgroups():
    """256 splits x 2 sequences x 2 head groups: each workgroup takes 4
    consecutive ranges of 64 tokens and merges them, so split g holds ranges
    4g .. 4g+3 (tokens [256 g, 256 g + 256)) and splits 64 .. 255 are empty;
    sequences of 3000 and 700 tokens leave most groups partly or wholly past
    the end.  Every sampled split against the oracle over its tokens."""
    lens = [3000, 700]
    S = 256
    wl = synth.workload("fp8_b1_l128k").with_(batch=2, heads=128, seq_len=None,
                                              seed=synth.workloads.BASE_SEED + 418)
    inp = synth.make_inputs(wl, lengths=lens)
    dev = DeviceInputs(inp)
    codes, scale = _query(2, 128, 419)
    _log("fp8 query multi-range")
    u, lse, u_part, lse_part = _decode(dev, codes, scale, S, part=torch.float32)
    pairs = [(b, h) for b in range(2) for h in (0, 64, 127)]
    e_u, e_l = _check(inp, codes, scale, u, lse, pairs)
    _log(f"  merged: err u {e_u:.2e} lse {e_l:.2e}")
    assert e_u <= TOL_FP8 and e_l <= TOL_FP8
    up, lp = u_part.cpu().numpy(), lse_part.cpu().numpy()
    R = ranges_per_split(2, 1, S, 128, grouped=True)
    assert R == 4
    chunk = 64 * R
    assert np.all(np.isneginf(lp[:, S // R:]))  # the slots past the groups
    for p in (0, 1, 2, 3, 10, 11, 12, 46, 47, 63):
        tb = [min(p * chunk, L) for L in lens]
        te = [min((p + 1) * chunk, L) for L in lens]
        u_ref, l_ref, _ = oracle.absorbed_decode(
            codes, "fp8", inp.rows, "fp8", inp.seq_lens, q_scale=scale, row_scale=inp.row_scale,
            seq_stride=inp.seq_stride, sel=pairs, t_begin=tb, t_end=te)
        for k, (b, h) in enumerate(pairs):
            if not np.isfinite(l_ref[k]):  # empty: lse = -inf, u not written
                assert np.isneginf(lp[b, p, h]), (p, b, h)
                continue
            assert abs(lp[b, p, h] - l_ref[k]) <= TOL_FP8, (p, b, h)
            assert _rel(up[b, p, h], u_ref[k]) <= TOL_FP8, (p, b, h)


def test_fp8_query_spike_inside_a_range_group():
    """A score spike in range 13 of 256 (ranges 12-15 share a workgroup and
    are merged into split 3): that group is computed again with its true
    maximum; its neighbours are not disturbed."""
    lens = [4000, 4000]
    S = 256
    wl = synth.workload("fp8_b1_l128k").with_(batch=2, heads=128, seq_len=None,
                                              seed=synth.workloads.BASE_SEED + 420)
    inp = synth.make_inputs(wl, lengths=lens)
    codes, scale = _query(2, 128, 421)
    q = oracle.decode_array(codes, "fp8")[0] * scale[0].astype(np.float64)[:, None]
    spike = np.sign(q.mean(axis=0)) * 40.0
    r = inp.row_index(0, 64 * 13 + 10)
    c8, s8 = quantize_rows_e4m3(spike[None, :].astype(np.float32))
    rows, rsc = inp.rows.copy(), inp.row_scale.copy()
    rows[r], rsc[r] = c8[0], s8[0]
    inp = dataclasses.replace(inp, rows=rows, row_scale=rsc)
    dev = DeviceInputs(inp)
    u, lse, u_part, lse_part = _decode(dev, codes, scale, S, part=torch.float32)
    pairs = [(b, h) for b in range(2) for h in (0, 77, 127)]
    up, lp = u_part.cpu().numpy(), lse_part.cpu().numpy()
    R = ranges_per_split(2, 1, S, 128, grouped=True)
    assert R == 4
    for p in (2, 3, 4):  # ranges 8-11, 12-15 (the spike), 16-19
        tb, te = [p * 64 * R] * 2, [(p + 1) * 64 * R] * 2
        u_ref, l_ref, _ = oracle.absorbed_decode(
            codes, "fp8", inp.rows, "fp8", inp.seq_lens, q_scale=scale, row_scale=inp.row_scale,
            seq_stride=inp.seq_stride, sel=pairs, t_begin=tb, t_end=te)
        for k, (b, h) in enumerate(pairs):
            assert abs(lp[b, p, h] - l_ref[k]) <= TOL_FP8, (p, b, h)
            assert _rel(up[b, p, h], u_ref[k]) <= TOL_FP8, (p, b, h)
    e_u, e_l = _check(inp, codes, scale, u, lse, pairs)
    _log(f"spike in a range group: err u {e_u:.2e} lse {e_l:.2e}")
    assert e_u <= TOL_FP8 and e_l <= TOL_FP8

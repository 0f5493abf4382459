"""GPU: the bf16 decode with many split ranges per sequence, where one
workgroup takes R consecutive ranges and merges them (R = the workgroups per
CU, capped at the split count, once there are 32 splits or more): split g
holds ranges gR .. gR+R-1 and the splits from ceil(S / R) on are empty.
Through the C ABI against the oracle's absorbed-form attention on the same
stored bf16 query:

* range groups that hold ranges past the end of a sequence, a group that
  straddles it, empty and one-token sequences;
* a split count that R does not divide (the last group is short);
* a paged cache with 64 heads;
* several query tokens per sequence (causal cut per token);
* a score spike in the middle of a range group: that group is computed
  again with its true maximum.
Every case checks the merged result and each sampled split's partial."""

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
from tests.mla_cases import ranges_per_split

pytestmark = pytest.mark.gpu

TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    assert np.all(np.isfinite(a)), "non-finite GPU output"
    return float(np.abs(a - b).max() / np.abs(b).max())


def _query(shape, seed):
    """absorbed query rows as bf16 bits: latent part N(0, 1/4), RoPE part N(0, 1)"""
    r = np.random.default_rng(seed)
    q = r.standard_normal(shape + (576,)).astype(np.float32)
    q[..., :512] *= 0.5
    return f32_to_bf16_bits(q)


def _chunk(max_len, S):
    return 32 * -(-max_len // (32 * S))


def _oracle(inp, q, pairs, t_begin=None, t_end=None):
    wl = inp.wl
    return oracle.absorbed_decode(
        q, "bf16", inp.rows, "bf16", inp.seq_lens, page_size=wl.page_size,
        seq_stride=inp.seq_stride, block_table=inp.block_table, sel=pairs,
        t_begin=t_begin, t_end=t_end)[:2]


def _check_partials(inp, q, up, lp, lens, S, splits, pairs, t_end_of=None, QL=1):
    """split p's partial against the oracle over tokens [p R chunk, (p+1) R
    chunk) (R ranges merged per split) cut at each sequence's attended
    length; the splits past the groups are empty"""
    H = q.shape[-2]
    R = ranges_per_split(inp.wl.batch, QL, S, H, grouped=S >= 32)
    chunk = _chunk(int(inp.max_seq_len), S) * R
    ng = -(-S // R)
    assert np.all(np.isneginf(lp[:, ng:]))
    att = np.asarray(lens if t_end_of is None else t_end_of)
    for p in splits:
        if p >= ng:
            continue
        tb = [int(min(p * chunk, L)) for L in att]
        te = [int(min((p + 1) * chunk, L)) for L in att]
        u_ref, l_ref = _oracle(inp, q, pairs, tb, te)
        for k, (b, h) in enumerate(pairs):
            if not np.isfinite(l_ref[k]):  # empty: lse = -inf, u not written
                assert np.isneginf(lp[b, p, h]), (p, b, h)
                continue
            assert abs(lp[b, p, h] - l_ref[k]) <= TOL, (p, b, h, lp[b, p, h], l_ref[k])
            assert _rel(up[b, p, h], u_ref[k]) <= TOL, (p, b, h)


def _run(dev, q, S):
    B, H = q.shape[0], q.shape[-2]
    u_part = torch.full((B, S, H, 512), float("nan"), dtype=torch.float32, device="cuda")
    lse_part = torch.full((B, S, H), float("nan"), dtype=torch.float32, device="cuda")
    mla.mla_decode(dev.geo, bits_to_tensor(q, "bf16"), dev.cache, S, u_part, lse_part)
    u = torch.empty(B, H, 512, dtype=torch.float32, device="cuda")
    lse = torch.empty(B, H, dtype=torch.float32, device="cuda")
    mla.mla_combine(dev.geo, u_part, lse_part, u, lse)
    torch.cuda.synchronize()
    return u.cpu().numpy(), lse.cpu().numpy(), u_part.cpu().numpy(), lse_part.cpu().numpy()


def _check_merged(inp, q, u, lse, pairs):
    u_ref, l_ref = _oracle(inp, q, pairs)
    u_got = np.stack([u[b, h] for b, h in pairs])
    l_got = np.array([lse[b, h] for b, h in pairs])
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isfinite(l_got), fin)
    assert np.all(u_got[~fin] == 0.0)
    return _rel(u_got[fin], u_ref[fin]), float(np.abs(l_got[fin] - l_ref[fin]).max())


CASES = [
    # name, lens, heads, S, page size, sampled splits
    # 8 x 64 splits x 2 head groups = 1024 range workgroups: R = 4, 16 splits written
    ("r4_ragged", [3000, 700, 1, 0, 1500, 64, 2047, 33], 128, 64, 0, (0, 1, 2, 3, 5, 10, 11, 15)),
    # 8 x 50 x 2 = 800: R = 3, 17 groups, the last of two ranges
    ("r3_short_last", [2000, 2000, 1999, 1601, 100, 100, 65, 1], 128, 50, 0, (0, 2, 3, 8, 15, 16)),
    # 16 x 32 x 1 = 512: R = 2, paged
    ("r2_paged_h64", [900, 1000, 1, 640, 128, 129, 500, 2] * 2, 64, 32, 64, (0, 1, 2, 7, 14, 15)),
]


@pytest.mark.parametrize("name,lens,H,S,ps,splits", CASES, ids=[c[0] for c in CASES])
def test_range_groups_match_the_oracle(name, lens, H, S, ps, splits):
    wl = synth.workload("dsv2_b32_l2k").with_(batch=len(lens), heads=H, seq_len=None,
                                              page_size=ps, seed=synth.workloads.BASE_SEED + 430)
    inp = synth.make_inputs(wl, lengths=lens)
    dev = DeviceInputs(inp)
    q = _query((len(lens), H), 431)
    _log(f"range groups {name} S={S}")
    u, lse, up, lp = _run(dev, q, S)
    pairs = [(b, h) for b in range(len(lens)) for h in sorted({0, 31, H // 2 + 5, H - 1})]
    e_u, e_l = _check_merged(inp, q, u, lse, pairs)
    _log(f"  merged: err u {e_u:.2e} lse {e_l:.2e}")
    assert e_u <= TOL and e_l <= TOL
    _check_partials(inp, q, up, lp, lens, S, splits, pairs)


def test_range_groups_several_query_tokens():
    """q_len = 3, 4 sequences, 32 splits, 128 heads: 4 x 3 x 32 x 2 = 768
    range workgroups, so R = 3 ranges merged per split (11 splits written);
    query token j attends the first L - (2 - j) rows."""
    lens = np.array([1200, 3, 700, 2], np.int32)
    B, QL, H, S = len(lens), 3, 128, 32
    wl = synth.workload("dsv2_b32_l2k").with_(batch=B, seq_len=None,
                                              seed=synth.workloads.BASE_SEED + 432)
    inp = synth.make_inputs(wl, lengths=lens.tolist())
    dev = DeviceInputs(inp)
    q = _query((B, QL, H), 433)
    u_part = torch.full((B, QL, S, H, 512), float("nan"), dtype=torch.float32, device="cuda")
    lse_part = torch.full((B, QL, S, H), float("nan"), dtype=torch.float32, device="cuda")
    _log("range groups q_len=3")
    mla.mla_decode_multi(dev.geo, bits_to_tensor(q, "bf16"), dev.cache, S, u_part, lse_part)
    torch.cuda.synchronize()
    up, lp = u_part.cpu().numpy(), lse_part.cpu().numpy()
    pairs = [(b, h) for b in range(B) for h in (0, 77, 127)]
    for j in range(QL):
        t_end = np.maximum(lens - (QL - 1 - j), 0)
        _check_partials(inp, q[:, j], up[:, j], lp[:, j], lens, S, (0, 1, 2, 3, 9, 10), pairs,
                        t_end_of=t_end, QL=QL)


def test_range_groups_spike_recomputes_one_range():
    """A score spike in range 13 of 256 (ranges of 64 tokens; ranges 12-15
    share a workgroup and are merged into split 3), far above the maximum of
    the group's first tile: the group is computed again with its true
    maximum, its neighbours keep their partials."""
    lens = [8200, 8200]
    S, H = 256, 128
    wl = synth.workload("dsv2_b32_l2k").with_(batch=2, seq_len=None,
                                              seed=synth.workloads.BASE_SEED + 434)
    inp = synth.make_inputs(wl, lengths=lens)
    q = _query((2, H), 435)
    chunk = _chunk(int(inp.max_seq_len), S)
    qf = q[0].view(np.uint16).astype(np.uint32) << 16
    qf = qf.view(np.float32).astype(np.float64)
    spike = np.sign(qf.mean(axis=0)) * 40.0
    rows = inp.rows.copy()
    assert chunk == 64
    rows[inp.row_index(0, 13 * chunk + 40)] = f32_to_bf16_bits(spike.astype(np.float32))
    inp = dataclasses.replace(inp, rows=rows)
    dev = DeviceInputs(inp)
    _log(f"range groups spike chunk={chunk}")
    u, lse, up, lp = _run(dev, q, S)
    pairs = [(b, h) for b in range(2) for h in (0, 77, 127)]
    u13, l13 = _oracle(inp, q, pairs[:3], [13 * chunk] * 2, [14 * chunk] * 2)
    first = _oracle(inp, q, pairs[:3], [12 * chunk] * 2, [12 * chunk + 32] * 2)[1]
    # some head's spike lies beyond the reference slack (the redo is taken for
    # the whole workgroup when any head's does)
    assert (l13 - first).max() > 64 / np.log2(np.e)
    assert ranges_per_split(2, 1, S, H, grouped=True) == 4
    _check_partials(inp, q, up, lp, lens, S, (2, 3, 4, 63, 64), pairs)
    e_u, e_l = _check_merged(inp, q, u, lse, pairs)
    _log(f"  merged: err u {e_u:.2e} lse {e_l:.2e}")
    assert e_u <= TOL and e_l <= TOL

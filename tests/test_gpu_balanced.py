"""GPU: the balanced partition of the bf16 decode (mla_decode_ex with
MLA_KERNEL_H64_BALANCED) through the C ABI against the oracle's
absorbed-form attention on the same stored bf16 query.

Every split of every row is checked, not only the merged result.  The
expected split boundaries come from tests.mla_cases.balanced_pieces, which
restates the partition rule of the C header.  The cases cover:
* a ragged paged batch with empty, one-token and long rows;
* several query tokens per sequence, each with its own causal cut;
* few tiles, where fewer workers than launched have a span;
* every row empty;
* 64 heads (256 workers of one workgroup each);
* a ring cache;
* the calls the partition does not take (fp8 cache, one split, more than
  512 rows)."""

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
from tests.mla_cases import balanced_pieces

pytestmark = pytest.mark.gpu

TOL = 2e-2
BAL = mla.KERNEL_H64_BALANCED


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


def _decode(dev, q, S, part=torch.float32):
    """balanced decode of q [B, h, 576] or [B, QL, h, 576]; partials as numpy"""
    lead = q.shape[:-2]
    H = q.shape[-2]
    u_part = torch.full((*lead, S, H, 512), float("nan"), dtype=part, device="cuda")
    lse_part = torch.full((*lead, S, H), float("nan"), dtype=torch.float32, device="cuda")
    mla.mla_decode_ex(dev.geo, bits_to_tensor(q, "bf16"), dev.cache, S, u_part, lse_part,
                      kernel=BAL)
    torch.cuda.synchronize()
    return u_part, lse_part


def _oracle_rows(inp, qb, b, rows, heads, ring):
    """oracle u, lse of sequence b over cache rows [rows[0], rows[1]) of its
    attended rows.  Rows are tokens, except in a ring that has wrapped: there
    the kernel attends the ring's rows in row order, row r holding the token
    t of the window [L - C, L) with t = r mod C.  Those tokens form at most two
    contiguous ranges, whose oracle results are merged by log-sum-exp."""
    L, C = int(inp.seq_lens[b]), int(inp.seq_stride)
    r0, r1 = rows
    if ring and L > C:
        toks = np.sort([L - C + ((r - (L - C)) % C) for r in range(r0, r1)])
        cut = np.flatnonzero(np.diff(toks) != 1) + 1
        runs = [(int(x[0]), int(x[-1]) + 1) for x in np.split(toks, cut)]
    else:
        runs = [(r0, r1)]
    parts = []
    for t0, t1 in runs:
        tb = np.zeros(inp.wl.batch, np.int32)
        te = np.zeros(inp.wl.batch, np.int32)
        tb[b], te[b] = t0, t1
        u, l, _ = oracle.absorbed_decode(
            qb, "bf16", inp.rows, "bf16", inp.seq_lens, page_size=inp.wl.page_size,
            seq_stride=inp.seq_stride, block_table=inp.block_table,
            sel=[(b, h) for h in heads], t_begin=tb, t_end=te, ring=ring)
        parts.append((u, l))
    if len(parts) == 1:
        return parts[0]
    (u1, l1), (u2, l2) = parts
    lse = np.logaddexp(l1, l2)
    return (np.exp(l1 - lse)[:, None] * u1 + np.exp(l2 - lse)[:, None] * u2), lse


def _check_splits(inp, q_rows, up, lp, att, S, HG, heads, ring=False):
    """every split of every row against the oracle over the split's tokens;
    q_rows [V, h, 576] and att[v] index rows v = b * QL + j, row v reading
    sequence v // QL of the cache"""
    V = len(att)
    QL = V // inp.wl.batch
    pieces = balanced_pieces(att, S, HG)
    up = up.float().cpu().numpy().reshape(V, S, -1, 512)
    lp = lp.cpu().numpy().reshape(V, S, -1)
    worst = 0.0
    for v in range(V):
        b = v // QL
        for p in range(S):
            rng = pieces[(v, p)]
            if rng is None:  # an empty split: lse = -inf (its u is not written)
                assert np.all(np.isneginf(lp[v, p, heads])), (v, p)
                continue
            qb = np.zeros((inp.wl.batch,) + q_rows.shape[1:], q_rows.dtype)
            qb[b] = q_rows[v]
            u_ref, l_ref = _oracle_rows(inp, qb, b, rng, heads, ring)
            assert np.all(np.abs(lp[v, p, heads] - l_ref) <= TOL), (v, p, rng)
            e = _rel(up[v, p, heads], u_ref)
            assert e <= TOL, (v, p, rng, e)
            worst = max(worst, e)
    return worst


CASES = [
    # name, lengths, heads, S, page size
    ("paged_ragged", [3000, 0, 1, 700, 16384, 33, 5000, 64, 0, 9000, 2, 12000], 128, 8, 64),
    ("contig_h64", [5000, 100, 0, 4097, 31, 2500], 64, 4, 0),
    ("few_tiles", [40, 1, 0, 64], 128, 8, 0),  # 5 tiles: 5 workers of 128 have spans
    ("two_splits", [1000, 1000, 3000, 0, 64], 128, 2, 0),  # G = N / n_max: few workers
]


@pytest.mark.parametrize("name,lens,H,S,ps", CASES, ids=[c[0] for c in CASES])
def test_balanced_splits_match_the_oracle(name, lens, H, S, ps):
    wl = synth.workload("paged_b64_ragged").with_(batch=len(lens), heads=H, seq_len=None,
                                                  page_size=ps, seed=synth.workloads.BASE_SEED + 440)
    inp = synth.make_inputs(wl, lengths=lens)
    dev = DeviceInputs(inp)
    q = _query((len(lens), H), 441)
    _log(f"balanced {name} S={S}")
    up, lp = _decode(dev, q, S)
    heads = sorted({0, 31, H // 2 + 3, H - 1})
    e = _check_splits(inp, q, up, lp, inp.seq_lens, S, (H + 63) // 64, heads)
    _log(f"  worst split err u {e:.2e}")
    # the merged result (mla_combine over the splits) against the whole range
    u = torch.empty(len(lens), H, 512, dtype=torch.float32, device="cuda")
    lse = torch.empty(len(lens), H, dtype=torch.float32, device="cuda")
    mla.mla_combine(dev.geo, up, lp, u, lse)
    torch.cuda.synchronize()
    pairs = [(b, h) for b in range(len(lens)) for h in heads]
    u_ref, l_ref, _ = oracle.absorbed_decode(
        q, "bf16", inp.rows, "bf16", inp.seq_lens, page_size=wl.page_size,
        seq_stride=inp.seq_stride, block_table=inp.block_table, sel=pairs)
    u, lse = u.cpu().numpy(), lse.cpu().numpy()
    fin = np.isfinite(l_ref)
    got_l = np.array([lse[b, h] for b, h in pairs])
    got_u = np.stack([u[b, h] for b, h in pairs])
    assert np.array_equal(np.isfinite(got_l), fin)
    assert np.all(got_u[~fin] == 0.0)
    assert _rel(got_u[fin], u_ref[fin]) <= TOL
    assert np.abs(got_l[fin] - l_ref[fin]).max() <= TOL


def test_balanced_every_row_empty():
    lens = [0, 0, 0]
    wl = synth.workload("paged_b64_ragged").with_(batch=3, seq_len=None, page_size=0,
                                                  seed=synth.workloads.BASE_SEED + 442)
    inp = synth.make_inputs(wl, lengths=lens, seq_stride=64)
    inp = dataclasses.replace(inp, max_seq_len=64)
    dev = DeviceInputs(inp)
    q = _query((3, 128), 443)
    _log("balanced: every row empty")
    up, lp = _decode(dev, q, 4, part=torch.bfloat16)
    assert torch.all(torch.isneginf(lp))


def test_balanced_several_query_tokens():
    """q_len = 3: rows v = b * 3 + j, row v attending L_b - (2 - j) tokens"""
    lens = np.array([2500, 2, 700, 0, 6000], np.int32)
    B, QL, H, S = len(lens), 3, 128, 6
    wl = synth.workload("paged_b64_ragged").with_(batch=B, seq_len=None,
                                                  seed=synth.workloads.BASE_SEED + 444)
    inp = synth.make_inputs(wl, lengths=lens.tolist())
    dev = DeviceInputs(inp)
    q = _query((B, QL, H), 445)
    _log("balanced q_len=3")
    up, lp = _decode(dev, q, S)
    att = [max(int(lens[b]) - (QL - 1 - j), 0) for b in range(B) for j in range(QL)]
    e = _check_splits(inp, q.reshape(B * QL, H, 576), up, lp, att, S, 2, [0, 77, 127])
    _log(f"  worst split err u {e:.2e}")


def test_balanced_ring_cache():
    """a ring of 1024 rows: sequences longer than the ring attend its 1024 rows"""
    C = 1024
    lens = [3000, 500, 1024, 1025, 7]
    wl = synth.workload("paged_b64_ragged").with_(batch=len(lens), seq_len=None, page_size=0,
                                                  seed=synth.workloads.BASE_SEED + 446)
    inp = synth.make_inputs(wl, lengths=[min(n, C) for n in lens], seq_stride=C)
    inp = dataclasses.replace(inp, seq_lens=np.asarray(lens, np.int32), max_seq_len=max(lens))
    dev = DeviceInputs(inp)
    dev.cache.ring = True
    q = _query((len(lens), 128), 447)
    _log("balanced ring")
    up, lp = _decode(dev, q, 4)
    att = [min(L, C) for L in lens]
    e = _check_splits(inp, q, up, lp, att, 4, 2, [0, 64, 127], ring=True)
    _log(f"  worst split err u {e:.2e}")


def test_balanced_refuses_what_it_does_not_take():
    wl = synth.workload("fp8_b1_l128k").with_(batch=2, seq_len=None,
                                              seed=synth.workloads.BASE_SEED + 448)
    inp = synth.make_inputs(wl, lengths=[100, 200])
    dev = DeviceInputs(inp)
    q = torch.zeros(2, 128, 576, dtype=torch.bfloat16, device="cuda")
    up = torch.empty(2, 4, 128, 512, dtype=torch.bfloat16, device="cuda")
    lp = torch.empty(2, 4, 128, dtype=torch.float32, device="cuda")
    with pytest.raises(mla.MLAError, match="not provided"):  # fp8 cache
        mla.mla_decode_ex(dev.geo, q, dev.cache, 4, up, lp, kernel=BAL)
    wl = synth.workload("paged_b64_ragged").with_(batch=513, seq_len=8, page_size=0,
                                                  seed=synth.workloads.BASE_SEED + 449)
    dev = DeviceInputs(synth.make_inputs(wl))
    q = torch.zeros(513, 128, 576, dtype=torch.bfloat16, device="cuda")
    up = torch.empty(513, 2, 128, 512, dtype=torch.bfloat16, device="cuda")
    lp = torch.empty(513, 2, 128, dtype=torch.float32, device="cuda")
    with pytest.raises(mla.MLAError, match="not provided"):  # more than 512 rows
        mla.mla_decode_ex(dev.geo, q, dev.cache, 2, up, lp, kernel=BAL)
    wl = synth.workload("paged_b64_ragged").with_(batch=4, seq_len=300, page_size=0,
                                                  seed=synth.workloads.BASE_SEED + 450)
    dev = DeviceInputs(synth.make_inputs(wl))
    up = torch.empty(4, 1, 128, 512, dtype=torch.bfloat16, device="cuda")
    lp = torch.empty(4, 1, 128, dtype=torch.float32, device="cuda")
    with pytest.raises(mla.MLAError, match="not provided"):  # one split
        mla.mla_decode_ex(dev.geo, q[:4].contiguous(), dev.cache, 1, up, lp, kernel=BAL)
    torch.cuda.synchronize()

"""Pins of the oracle's absorbed-form attention (oracle_absorbed_decode) and of
its E4M3 row quantiser (oracle_quantize_e4m3_rows), which check the fp8
absorbed query of the 128K fp8 workload.

* The absorbed identity of the DeepSeek V2 MLA page (section 2.3): with the
  oracle's own absorbed query (oracle_absorb_q, float64) the absorbed form
  reproduces the naive rebuild decode (oracle_mla_decode) -- u, lse and o --
  on contiguous, paged and ring caches, bf16 and fp8 rows, and sub-ranges.
* Closed forms: one attended token gives its latent; a zero query gives the
  plain mean of the latents and lse = log n.
* The E4M3 query factor: codes with their factor equal the decoded values
  passed as float64; doubling the factor doubles every score.
* The quantiser equals an independent numpy quantiser (the one the synthetic
  fp8 cache rows are made with) code for code, and the cache append's E4M3
  rows.
"""

import math

import numpy as np
import pytest

import oracle
import synth
from synth.encode import quantize_rows_e4m3

TIGHT = 1e-12


def _inputs(name, lens, heads=8, seed=0, **kw):
    wl = synth.workload(name).with_(batch=len(lens), heads=heads, seq_len=None,
                                    seed=synth.workloads.BASE_SEED + 300 + seed, **kw)
    return synth.make_inputs(wl, lengths=lens)


def _absorbed(inp, q_abs, q_dt="f64", q_scale=None, **kw):
    wl = inp.wl
    return oracle.absorbed_decode(q_abs, q_dt, inp.rows, wl.cache_dtype, inp.seq_lens,
                                  q_scale=q_scale, row_scale=inp.row_scale,
                                  page_size=wl.page_size, seq_stride=inp.seq_stride,
                                  block_table=inp.block_table, d_nope=wl.d_nope,
                                  w_uv=inp.w_uv, w_dtype=wl.act_dtype, **kw)


def _rel(a, b):
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-300))


@pytest.mark.parametrize("name,kw", [("dsv2_b32_l2k", {}), ("dsv2_b32_l2k", {"page_size": 64}),
                                     ("fp8_b1_l128k", {})])
def test_absorbed_form_reproduces_the_naive_decode(name, kw):
    lens = [130, 64, 1, 0]
    inp = _inputs(name, lens, seed=1, **kw)
    wl = inp.wl
    qa = oracle.absorb_q(inp.q_nope, inp.q_rope, wl.act_dtype, inp.w_uk, wl.act_dtype)
    u, lse, o = _absorbed(inp, qa)
    o_n, lse_n, u_n = oracle.decode_inputs(inp, want_u=True)
    assert _rel(u, u_n) <= TIGHT and _rel(o, o_n) <= TIGHT
    fin = np.isfinite(lse_n)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.abs(lse[fin] - lse_n[fin]).max() <= TIGHT
    assert np.all(u[~np.repeat(fin, 1)] == 0.0)  # empty sequence: u = 0, lse = -inf


def test_sub_ranges_and_ring_follow_the_naive_decode():
    lens = [200, 90]
    inp = _inputs("dsv2_b32_l2k", lens, seed=2)
    wl = inp.wl
    qa = oracle.absorb_q(inp.q_nope, inp.q_rope, wl.act_dtype, inp.w_uk, wl.act_dtype)
    tb, te = [17, 0], [150, 33]
    u, lse, _ = _absorbed(inp, qa, t_begin=tb, t_end=te)
    _, lse_n, u_n = oracle.decode_inputs(inp, want_u=True, t_begin=tb, t_end=te)
    assert _rel(u, u_n) <= TIGHT and np.abs(lse - lse_n).max() <= TIGHT
    # a ring of 64 slots holding the last 64 of 200 and 90 tokens
    C = 64
    ring_inp = synth.make_inputs(wl, lengths=[C, C], seq_stride=C)
    import dataclasses
    ring_inp = dataclasses.replace(ring_inp, seq_lens=np.asarray(lens, np.int32))
    u_r, lse_r, _ = _absorbed(ring_inp, qa, ring=True)
    _, lse_rn, u_rn = oracle.decode_inputs(ring_inp, want_u=True, ring=True)
    assert _rel(u_r, u_rn) <= TIGHT and np.abs(lse_r - lse_rn).max() <= TIGHT


def test_closed_forms():
    inp = _inputs("dsv2_b32_l2k", [1, 40], heads=4, seed=3)
    rows = oracle.decode_array(inp.rows, "bf16")
    qa = np.random.default_rng(5).standard_normal((2, 4, 576))
    qa[1] = 0.0  # zero query on sequence 1
    u, lse, _ = _absorbed(inp, qa)
    u = u.reshape(2, 4, 512)
    lse = lse.reshape(2, 4)
    r0 = rows[inp.row_index(0, 0)]
    scale = 1.0 / math.sqrt(192.0)
    for h in range(4):
        assert np.array_equal(u[0, h], r0[:512])  # one token: its latent, weight 1
        assert abs(lse[0, h] - scale * float(qa[0, h] @ r0)) <= 1e-12 * max(1.0, abs(lse[0, h]))
    mean = np.mean([rows[inp.row_index(1, t)][:512] for t in range(40)], axis=0)
    assert _rel(u[1], np.broadcast_to(mean, (4, 512))) <= TIGHT
    assert np.abs(lse[1] - math.log(40)).max() <= TIGHT


def test_e4m3_query_is_codes_times_its_factor():
    """The factor of (b, h) multiplies that row's codes: codes + factors equal
    the decoded values given as float64, and a doubled factor doubles every
    score, so lse - m scales exactly as for a query twice as large."""
    inp = _inputs("fp8_b1_l128k", [70, 33, 5], heads=4, seed=4)
    rng = np.random.default_rng(6)
    x = (rng.standard_normal((3, 4, 576)) * rng.uniform(0.1, 10, (3, 4, 1))).astype(np.float32)
    codes, scale = oracle.quantize_e4m3_rows(x)
    assert len(np.unique(scale)) == scale.size  # distinct factors: an index mix-up shows
    dq = oracle.decode_array(codes, "fp8") * scale.astype(np.float64)[..., None]
    u8, l8, o8 = _absorbed(inp, codes, "fp8", q_scale=scale)
    u64, l64, o64 = _absorbed(inp, dq)
    assert np.array_equal(u8, u64) and np.array_equal(l8, l64) and np.array_equal(o8, o64)
    u2, _, _ = _absorbed(inp, codes, "fp8", q_scale=2 * scale)
    u2d, _, _ = _absorbed(inp, 2 * dq)
    assert np.array_equal(u2, u2d) and _rel(u2, u8) > 1e-6


def test_quantiser_equals_an_independent_one_and_the_cache_rows():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((40, 576)).astype(np.float32) * rng.uniform(1e-3, 1e3, (40, 1)).astype(np.float32)
    x[3] = 0.0                      # all-zero row: factor 2^-126 / 448, codes 0
    x[4, :7] = [448, -448, 1e-30, -1e-30, 3.5, 3.75, -0.0]
    x[5, -1] = -1e4                 # the row's largest magnitude in its last element
    x[6, 0] = 1e4                   # ... and in its first
    codes, scale = oracle.quantize_e4m3_rows(x)
    c_ref, s_ref = quantize_rows_e4m3(x)
    assert np.array_equal(codes, c_ref) and np.array_equal(scale.view(np.uint32), s_ref.view(np.uint32))
    assert np.all(codes[3] == 0) and scale[3] == np.float32(2.0 ** -126) / np.float32(448)
    # the cache append stores the same codes and factors
    rows = np.zeros((41, 576), np.uint8)  # one guard row
    rs = np.zeros(41, np.float32)
    oracle.cache_append(x[:, :512], x[:, 512:], "f32", np.zeros(40, np.int32), rows, "fp8",
                        row_scale=rs, seq_stride=1)
    assert np.array_equal(rows[:40], codes) and np.array_equal(rs[:40], scale)


def test_absorb_q_fp8_is_the_quantised_absorbed_query():
    inp = _inputs("fp8_b1_l128k", [10], heads=4, seed=9)
    wl = inp.wl
    codes, scale = oracle.absorb_q_fp8(inp.q_nope, inp.q_rope, wl.act_dtype, inp.w_uk, wl.act_dtype)
    qa = oracle.absorb_q(inp.q_nope, inp.q_rope, wl.act_dtype, inp.w_uk, wl.act_dtype)
    dq = oracle.decode_array(codes, "fp8") * scale.astype(np.float64)[..., None]
    # every value within half an E4M3 step (2^-4 relative, or 2^-10 of the
    # factor near zero) of the float64 absorbed query
    step = np.maximum(np.abs(qa) * 2.0 ** -4, scale.astype(np.float64)[..., None] * 2.0 ** -10)
    assert np.all(np.abs(dq - qa) <= step * (1 + 1e-6))
    amax = np.abs(qa.astype(np.float32)).max(axis=-1)
    assert np.array_equal(scale, (amax / np.float32(448)).astype(np.float32))

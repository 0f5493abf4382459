"""Pins of the oracle's naive-form rebuild ([V2] §2.1: every head's key
W_UK c_t concatenated with the shared k_R,t, and value W_UV c_t) that the
chunked-prefill path is checked against: the rebuilt keys and values, run
through the multi-head attention oracle (itself pinned to torch SDPA), give
the MLA decode oracle (pinned to SDPA over its own rebuild); a sub-range is
the slice of the whole; paged equals contiguous.  The causal prefill reading
(query token j of a chunk of n at the end of a length-L cache attends tokens
0 .. L - n + j, [LAT] §4.2's causal varlen call) is the decode oracle with a
per-query end, which the last test ties to the multi-head oracle on a causal
prefix."""

import numpy as np
import pytest

import oracle
import synth


def _inp(page_size=0, lens=(50, 7), seed=170):
    wl = synth.workload("dsv2_b32_l2k").with_(batch=len(lens), heads=4, seq_len=None,
                                             page_size=page_size,
                                             seed=synth.workloads.BASE_SEED + seed)
    return synth.make_inputs(wl, lengths=list(lens))


def test_rebuilt_keys_and_values_reproduce_the_decode():
    inp = _inp()
    lens = inp.seq_lens
    H, Lm = 4, int(lens.max())
    K = np.zeros((2, H, Lm, 192))
    V = np.zeros((2, H, Lm, 128))
    for b, L in enumerate(lens):
        K[b, :, :L], V[b, :, :L] = oracle.rebuild_kv_inputs(inp, b, 0, int(L))
    q = np.concatenate([oracle.decode_array(inp.q_nope, "bf16"),
                        oracle.decode_array(inp.q_rope, "bf16")], axis=-1)
    o, lse = oracle.mha_decode(q, K, V, "f64", lens, scale=1 / np.sqrt(192.0))
    o_ref, lse_ref, _ = oracle.decode_inputs(inp)
    assert np.allclose(o.reshape(-1, 128), o_ref, rtol=0, atol=1e-12)
    assert np.allclose(lse.ravel(), lse_ref, rtol=0, atol=1e-12)


def test_sub_range_is_a_slice_and_paged_equals_contiguous():
    c, p = _inp(), _inp(page_size=64)
    kf, vf = oracle.rebuild_kv_inputs(c, 0, 0, 50)
    ks, vs = oracle.rebuild_kv_inputs(c, 0, 13, 41)
    assert np.array_equal(ks, kf[:, 13:41]) and np.array_equal(vs, vf[:, 13:41])
    kp, vp = oracle.rebuild_kv_inputs(p, 0, 0, 50)
    assert np.array_equal(kp, kf) and np.array_equal(vp, vf)
    # the RoPE half of every head's key is the token's cached k_R
    rows = oracle.decode_array(c.rows, "bf16")
    assert np.array_equal(kf[2, 5, 128:], rows[c.row_index(0, 5), 512:])


def test_causal_chunk_is_the_decode_with_a_per_query_end():
    """A chunk of n = 5 queries at the end of a 30-token cache: query j's
    decode over tokens [0, 30 - 5 + j] equals multi-head attention over the
    rebuilt keys and values cut at that token."""
    inp = _inp(lens=(30,), seed=171)
    k, v = oracle.rebuild_kv_inputs(inp, 0, 0, 30)
    r = np.random.default_rng(3)
    n = 5
    qn = r.standard_normal((n, 4, 128))
    qr = r.standard_normal((n, 4, 64))
    for j in range(n):
        end = 30 - n + j + 1
        o_ref, lse_ref, _ = oracle.decode(qn[j:j + 1], qr[j:j + 1], "f64", inp.w_uk, inp.w_uv,
                                          "bf16", inp.rows, "bf16", inp.seq_lens,
                                          seq_stride=inp.seq_stride, t_end=[end])
        q = np.concatenate([qn[j], qr[j]], -1)[None]
        o, lse = oracle.mha_decode(q, k[None, :, :end], v[None, :, :end], "f64",
                                   np.array([end], np.int32), scale=1 / np.sqrt(192.0))
        assert np.allclose(o.reshape(-1, 128), o_ref, rtol=0, atol=1e-12)
        assert np.allclose(lse.ravel(), lse_ref, rtol=0, atol=1e-12)

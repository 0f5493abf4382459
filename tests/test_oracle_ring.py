"""Pins of the oracle's ring cache ([V2] §4.1: the KV cache is kept in a ring
buffer so that it can grow).  Reading: a sequence's seq_stride rows form a ring
of capacity C; token t is written into row t mod C, so the ring holds the last
min(L, C) tokens and the decode attends those (a window of C tokens once
L > C); growing the ring moves that window into a ring of capacity C', token t
to row t mod C'.  The pins tie the ring to the linear cache (itself pinned to
library attention): appending tokens one by one into a ring and decoding it
gives the linear decode over the last C tokens."""

import numpy as np
import pytest

import oracle
from .test_oracle_pins import assert_close

DN, DR, DL, DV, H = 16, 8, 32, 12, 3
W = DL + DR


def _weights(rng, B):
    return dict(q_nope=rng.standard_normal((B, H, DN)), q_rope=rng.standard_normal((B, H, DR)),
                w_uk=rng.standard_normal((H, DN, DL)) / np.sqrt(DL),
                w_uv=rng.standard_normal((H, DV, DL)) / np.sqrt(DL))


def _decode(p, rows, lens, stride, ring=False, t_begin=None):
    return oracle.decode(p["q_nope"], p["q_rope"], "f64", p["w_uk"], p["w_uv"], "f64", rows, "f64",
                         np.asarray(lens, np.int32), seq_stride=stride, ring=ring,
                         t_begin=t_begin, want_u=True)


def _ring_by_appends(tokens, C, lens=None):
    """the first lens[b] tokens of tokens [B, L, W] (float32) appended one
    position at a time into rings of capacity C (f32 cache); a position -1
    skips a sequence that is already complete"""
    B, L, _ = tokens.shape
    lens = [L] * B if lens is None else lens
    # unwritten slots hold NaN, which would poison a decode that read them; a
    # guard row past the end keeps a wrong row map inside the array
    rows = np.full((B * C + 1, W), np.nan, np.float32)
    for t in range(L):
        pos = np.array([t if t < n else -1 for n in lens], np.int32)
        oracle.cache_append(tokens[:, t, :DL], tokens[:, t, DL:], "f32", pos, rows, "f32",
                            seq_stride=C, ring=True)
    return rows[:B * C]


@pytest.mark.parametrize("L,C", [(20, 32), (32, 32), (45, 32), (100, 16), (64, 7)])
def test_ring_decode_is_the_linear_decode_over_the_last_c_tokens(L, C):
    rng = np.random.default_rng(L * 100 + C)
    B = 2
    p = _weights(rng, B)
    tokens = rng.standard_normal((B, L, W)).astype(np.float32)
    ring = _ring_by_appends(tokens, C)
    linear = tokens.reshape(B * L, W).astype(np.float64)
    o_r, l_r, u_r = _decode(p, ring.astype(np.float64), [L] * B, C, ring=True)
    t0 = max(0, L - C)
    o_l, l_l, u_l = _decode(p, linear, [L] * B, L, t_begin=[t0] * B)
    assert_close(o_r, o_l)
    assert_close(u_r, u_l)
    assert_close(l_r, l_l)
    # the rows themselves: token t in row t mod C for the live window
    for b in range(B):
        for t in range(t0, L):
            assert np.array_equal(ring[b * C + t % C], tokens[b, t])


def test_ring_within_capacity_equals_the_linear_cache_bit_for_bit():
    rng = np.random.default_rng(5)
    B, L, C = 3, 40, 64
    p = _weights(rng, B)
    rows = rng.standard_normal((B * C, W))
    lens = [40, 1, 0]
    a = _decode(p, rows, lens, C, ring=True)
    b = _decode(p, rows, lens, C)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("C,C2,lens", [(16, 48, [12, 16, 0]), (16, 16, [50, 9, 0]),
                                        (32, 8, [50, 9, 0])])
def test_grown_ring_decodes_like_the_window_it_keeps(C, C2, lens):
    """Growing moves the live window, token t to row t mod C2.  A ring grown
    before it wrapped (L <= C) has lost nothing: appending the following
    tokens into the grown ring and decoding it gives the linear decode over
    all of them while they fit.  Shrinking keeps the last C2 tokens: it decodes
    like the linear cache from L - C2."""
    rng = np.random.default_rng(C * 7 + C2)
    B, L = 3, 50
    p = _weights(rng, B)
    tokens = rng.standard_normal((B, L, W)).astype(np.float32)
    ring = _ring_by_appends(tokens, C, lens)
    scale = rng.standard_normal(B * C).astype(np.float32)
    grown, gscale = oracle.ring_grow(lens, ring, C, C2, src_scale=scale)
    for b in range(B):
        keep = min(lens[b], C, C2)
        for t in range(lens[b] - keep, lens[b]):
            assert np.array_equal(grown[b * C2 + t % C2], ring[b * C + t % C])
            assert gscale[b * C2 + t % C2] == scale[b * C + t % C]
    final = list(lens)
    if C2 > C:  # keep appending into the grown ring, up to its capacity
        final = [min(C2, n + 20) if n else 0 for n in lens]
        grown = grown.astype(np.float32)
        for t in range(max(final)):
            pos = np.array([t if n <= t < f else -1 for n, f in zip(lens, final)], np.int32)
            oracle.cache_append(tokens[:, t, :DL], tokens[:, t, DL:], "f32", pos, grown, "f32",
                                seq_stride=C2, ring=True)
    o_g, l_g, u_g = _decode(p, grown.astype(np.float64), final, C2, ring=True)
    linear = tokens.reshape(B * L, W).astype(np.float64)
    o_r, l_r, u_r = _decode(p, linear, final, L, t_begin=[max(0, n - min(C, C2) if C2 <= C else 0)
                                                          for n in final])
    assert_close(o_g, o_r, 1e-12)
    assert_close(u_g, u_r, 1e-12)
    fin = np.isfinite(l_r)
    assert np.array_equal(fin, np.isfinite(l_g)) and np.abs(l_g[fin] - l_r[fin]).max() < 1e-12

"""Pins of the oracle's decoupled RoPE of q_R ([V2] §2.2: the positional
query and key are rotated, the content query is not; [LAT]'s rotary listing:
frequencies 1/10000^(2i/d), the d/2 angles repeated over both halves).  The
pins: position 0 is the identity; each (i, i + d/2) pair keeps its length; the
pages' listing form (cat(freqs, freqs), x*cos + rotate_half(x)*sin) written
out in numpy; the relative-position property of rotary embeddings; the
frequency table's end points."""

import numpy as np
import pytest

import oracle

D = 64


def _x(seed, B=3, H=5):
    return np.random.default_rng(seed).standard_normal((B, H, D)).astype(np.float32)


def test_inverse_frequencies():
    f = oracle.rope_inv_freq(D, 10000.0).astype(np.float64)
    assert f[0] == 1.0
    assert f[16] == np.float32(0.01)           # 10000^(-32/64)
    assert np.all(np.diff(f) < 0)
    assert np.allclose(f, 10000.0 ** (-np.arange(0, D, 2) / D), rtol=2 ** -24, atol=0)


def test_position_zero_is_the_identity():
    x = _x(1)
    out = oracle.rope(x, "f32", np.zeros(3, np.int32))
    assert np.array_equal(out, x.astype(np.float64))


@pytest.mark.parametrize("pos", [1, 17, 2048, 131071])
def test_pairs_keep_their_length(pos):
    x = _x(2)
    out = oracle.rope(x, "f32", np.full(3, pos, np.int32))
    h = D // 2
    n_in = np.hypot(x[..., :h].astype(np.float64), x[..., h:].astype(np.float64))
    n_out = np.hypot(out[..., :h], out[..., h:])
    assert np.allclose(n_in, n_out, rtol=1e-14, atol=1e-14)


def _listing_form(x, pos, base=10000.0):
    """The [LAT] rotary listing in numpy: inv_freq, outer product with the
    positions in float32, cat(freqs, freqs), x*cos + rotate_half(x)*sin with
    rotate_half(x) = cat(-x2, x1); the cos/sin taken in float64."""
    inv = oracle.rope_inv_freq(D, base)
    freqs = (np.asarray(pos, np.float32)[:, None] * inv[None, :]).astype(np.float32)
    emb = np.concatenate([freqs, freqs], axis=-1).astype(np.float64)[:, None, :]
    x = x.astype(np.float64)
    rot = np.concatenate([-x[..., D // 2:], x[..., :D // 2]], axis=-1)
    return x * np.cos(emb) + rot * np.sin(emb)


def test_matches_the_listing_form():
    x = _x(3)
    pos = np.array([3, 1000, 131071], np.int32)
    assert np.allclose(oracle.rope(x, "f32", pos), _listing_form(x, pos), rtol=0, atol=1e-12)
    assert np.allclose(oracle.rope(x, "f32", pos, base=500.0), _listing_form(x, pos, 500.0),
                       rtol=0, atol=1e-12)


def test_scores_depend_on_the_relative_position():
    """<R(m) q, R(n) k> = <q, R(n - m) k> for rotary embeddings; with angles
    rounded to binary32 it holds to the angle rounding at these positions."""
    q, k = _x(4, 1, 1), _x(5, 1, 1)
    for m, n in [(0, 7), (5, 12), (100, 107), (1000, 1007)]:
        a = np.dot(oracle.rope(q, "f32", np.array([m], np.int32)).ravel(),
                   oracle.rope(k, "f32", np.array([n], np.int32)).ravel())
        b = np.dot(q.astype(np.float64).ravel(),
                   oracle.rope(k, "f32", np.array([n - m], np.int32)).ravel())
        assert abs(a - b) < 1e-4 * np.linalg.norm(q) * np.linalg.norm(k), (m, n)


def test_heads_share_the_sequence_position():
    x = _x(6, B=2, H=4)
    out = oracle.rope(x, "f32", np.array([9, 33], np.int32))
    for h in range(4):
        one = oracle.rope(x[:, h:h + 1], "f32", np.array([9, 33], np.int32))
        assert np.array_equal(out[:, h:h + 1], one)

"""Pins of the oracle's decoupled RoPE of q_R ([V2] §2.2: the positional
query and key are rotated, the content query is not; [LAT]'s rotary listing:
frequencies 1/10000^(2i/d), element i paired with i + d/2).  The pins come from
the rotation itself: position 0 is the identity; each (i, i + d/2) pair keeps
its length; the angle read back from the output with atan2 is the binary32
product position x inv_freq[i], turning counter-clockwise, and no other element
moves; pair 0 (inv_freq = 1) turns by the position in radians (quarter-turn
closed forms); angles add; the relative-position property of rotary scores;
the frequency table's end points."""

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


def _unit_rows(i):
    """x[0, 0] = e_i: the rotation's column i"""
    x = np.zeros((1, 1, D), np.float32)
    x[0, 0, i] = 1.0
    return x


@pytest.mark.parametrize("pos", [1, 11, 1000, 131071])
def test_rotation_angle_is_the_binary32_product(pos):
    """e_i goes to cos(theta) e_i + sin(theta) e_(i+d/2), and e_(i+d/2) to
    -sin(theta) e_i + cos(theta) e_(i+d/2): a counter-clockwise turn of the
    (i, i + d/2) plane and nothing else.  The angle, read back with atan2 from
    the output, is the binary32 product position x inv_freq[i] (reading of
    [V2] §2.2 with the angle precision of the listings).  At 131071 the binary32
    rounding of the angle is ~1e-3 rad, far above the tolerance, so a double
    angle fails; so does a turn the other way or another pairing."""
    inv = oracle.rope_inv_freq(D, 10000.0)
    h = D // 2
    for i in range(h):
        theta = float(np.float32(pos) * inv[i])  # numpy float32 product: IEEE round to nearest
        for col, (a, b) in ((i, (1.0, 0.0)), (i + h, (0.0, 1.0))):
            out = oracle.rope(_unit_rows(col), "f32", np.array([pos], np.int32))[0, 0]
            others = np.delete(out, [i, i + h])
            assert np.all(others == 0.0), (pos, col)
            # the image of (a, b) in the (i, i+h) plane, turned back by theta
            got = np.arctan2(out[i + h], out[i]) - np.arctan2(b, a)
            d = (got - theta + np.pi) % (2 * np.pi) - np.pi
            assert abs(d) < 1e-9, (pos, col, d)
            assert abs(np.hypot(out[i], out[i + h]) - 1.0) < 1e-15


def test_quarter_turns_of_the_unit_frequency_pair():
    """Pair 0 has inv_freq = 1 exactly, so it turns by the position in radians:
    11 rad is within 5e-3 rad of three quarter turns (3 pi / 2) and 8 rad of two
    and a half; the images of e_0 are then close to -e_32 and to e_32, and
    the closed forms cos(p), sin(p) hold."""
    for pos, want in ((11, (0.0, -1.0)), (8, (-0.1455, 0.9894))):
        out = oracle.rope(_unit_rows(0), "f32", np.array([pos], np.int32))[0, 0]
        assert abs(out[0] - np.cos(pos)) < 1e-15 and abs(out[32] - np.sin(pos)) < 1e-15
        assert abs(out[0] - want[0]) < 5e-3 and abs(out[32] - want[1]) < 5e-3


@pytest.mark.parametrize("a,b", [(3, 4), (100, 28), (1000, 24)])
def test_angles_add(a, b):
    """Turning by position a and then by b is turning by a + b, up to the
    binary32 rounding of the three angles."""
    x = _x(3)
    once = oracle.rope(x, "f32", np.full(3, a + b, np.int32))
    ya = oracle.rope(x, "f32", np.full(3, a, np.int32)).astype(np.float32)
    twice = oracle.rope(ya, "f32", np.full(3, b, np.int32))
    tol = 4 * (a + b) * 2.0 ** -24 * np.abs(x).max() + 1e-6
    assert np.abs(twice - once).max() < tol


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

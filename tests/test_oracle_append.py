"""Pins of the oracle's cache append (the step before decode: one new token's
[c_KV | k_R] row per sequence, [V2] §2.3, kept in FP8 for long contexts per
[DSA]).  Each pin ties it to something other than itself: the E4M3 decode
table and the OCP spacing rules, the independent numpy quantiser that makes
the stored inputs (synth.encode), the bf16 rounding of the same module, and
the row map of the decode oracle."""

import numpy as np
import pytest

import oracle
import synth
from synth.encode import f32_to_bf16_bits, quantize_rows_e4m3

W = 576  # d_latent + d_rope
DL, DR = 512, 64


def _append_rows(x, src, cache):
    """Append row b of x (binary32 [n, W], or bf16 bits for src "bf16") as
    token 0 of sequence b (seq_stride 1); one guard row past the end keeps a
    wrong row map inside the arrays.  Returns (rows[:n], scales[:n] or None)."""
    n = x.shape[0]
    npdt = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}[cache]
    rows = np.zeros((n + 1, W), dtype=npdt)
    rs = np.zeros(n + 1, dtype=np.float32) if cache == "fp8" else None
    oracle.cache_append(x[:, :DL], x[:, DL:], src, np.zeros(n, np.int32), rows, cache,
                        row_scale=rs, seq_stride=1)
    return rows[:n], (None if rs is None else rs[:n])


def _finite_codes():
    return [c for c in range(256) if (c & 0x7F) != 0x7F]


def _value(code):
    return float(oracle.lib().oracle_decode_e4m3(code))


def test_e4m3_encode_returns_every_code_of_its_value():
    for c in _finite_codes():
        got = oracle.encode_e4m3(np.float32(_value(c)))
        # +0 and -0 keep their sign bit
        assert got == c, (hex(c), hex(got))


def test_e4m3_encode_ties_go_to_the_even_mantissa():
    """Between two neighbouring codes of one sign, the midpoint goes to the
    code with an even mantissa (LSB 0), values just inside go to the nearer;
    this covers the subnormal/normal seam (7.5 x 2^-9) and every binade seam."""
    pos = sorted((_value(c), c) for c in _finite_codes() if c < 0x80 and c != 0x00)
    pos = [(0.0, 0x00)] + pos
    for (v0, c0), (v1, c1) in zip(pos, pos[1:]):
        mid = np.float32((v0 + v1) / 2)
        assert float(mid) == (v0 + v1) / 2  # midpoints are binary32 values
        want = c0 if (c0 & 1) == 0 else c1
        assert oracle.encode_e4m3(mid) == want, (v0, v1)
        assert oracle.encode_e4m3(-mid) == want | 0x80
        below = np.nextafter(mid, np.float32(0))
        above = np.nextafter(mid, np.float32(np.inf))
        assert oracle.encode_e4m3(below) == c0
        assert oracle.encode_e4m3(above) == c1


def test_e4m3_encode_saturates_at_448():
    assert oracle.encode_e4m3(np.float32(448.0)) == 0x7E
    assert oracle.encode_e4m3(np.float32(460.0)) == 0x7E
    assert oracle.encode_e4m3(np.float32(-1000.0)) == 0xFE


def _rows(seed, n, spread):
    r = np.random.default_rng(seed)
    x = r.standard_normal((n, W)).astype(np.float32)
    # per-row magnitudes across the binary32 range, and rows with exact zeros
    x *= (10.0 ** r.uniform(-spread, spread, size=(n, 1))).astype(np.float32)
    x[:, ::37] = 0.0
    return x


@pytest.mark.parametrize("spread", [0.0, 3.0, 30.0])
def test_fp8_append_matches_the_input_quantiser(spread):
    """The stored fp8 inputs come from synth.encode.quantize_rows_e4m3 (numpy,
    a separate implementation of the same rule); appending the same binary32
    rows must give the same codes and the same scales, bit for bit."""
    n = 64
    x = _rows(11 + int(spread), n, spread)
    x[5] = 0.0  # all-zero row: scale 2^-126 / 448, every code 0
    codes, scales = quantize_rows_e4m3(x)
    rows, rs = _append_rows(x, "f32", "fp8")
    assert np.array_equal(rows, codes)
    assert np.array_equal(rs.view(np.uint32), scales.view(np.uint32))


def test_fp8_append_dequantises_within_half_a_spacing():
    x = _rows(3, 16, 2.0)
    rows, rs = _append_rows(x, "f32", "fp8")
    back = oracle.decode_array(rows, "fp8") * rs[:, None].astype(np.float64)
    y = x.astype(np.float64)
    # relative spacing of E4M3 is 2^-3 (normal), so |error| <= 2^-4 |y| + half the
    # subnormal spacing (2^-10 in units of the scale)
    assert np.all(np.abs(back - y) <= 2.0 ** -4 * np.abs(y) + 2.0 ** -10 * rs[:, None] + 1e-45)
    # the row maximum is exactly 448 * scale
    amax = np.max(np.abs(back), axis=1)
    assert np.array_equal(amax, 448.0 * rs.astype(np.float64))


def test_bf16_append_rounds_to_nearest_even():
    r = np.random.default_rng(5)
    x = r.standard_normal((8, W)).astype(np.float32)
    # exact ties: low 16 bits 0x8000 with even and odd upper halves
    u = x.view(np.uint32)
    u[:, :16] = (u[:, :16] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    rows, _ = _append_rows(x, "f32", "bf16")
    assert np.array_equal(rows, f32_to_bf16_bits(x))


def test_f32_and_bf16_inputs_are_stored_exactly():
    r = np.random.default_rng(6)
    x = r.standard_normal((4, W)).astype(np.float32)
    rows, _ = _append_rows(x, "f32", "f32")
    assert np.array_equal(rows.view(np.uint32), x.view(np.uint32))
    b = f32_to_bf16_bits(x)
    rows16, _ = _append_rows(b, "bf16", "bf16")
    assert np.array_equal(rows16, b)
    rows32, _ = _append_rows(b, "bf16", "f32")
    assert np.array_equal(rows32, synth.bf16_bits_to_f32(b))


def test_append_places_rows_like_the_decode_row_map():
    """The appended row of (b, t) is the row the decode oracle reads for token
    t of sequence b (contiguous and paged); nothing else changes, and
    positions < 0 or past the capacity are skipped."""
    B, ps, max_pages = 5, 64, 3
    r = np.random.default_rng(9)
    perm = r.permutation(B * max_pages).astype(np.int32).reshape(B, max_pages)
    x = r.standard_normal((B, W)).astype(np.float32)
    # sequence 1 asks for a position past its capacity (3 pages; stride 10): a
    # row map that ignored the capacity would land in sequence 2's rows, which
    # the check below sees, rather than outside the arrays
    pos = np.array([0, 192, 64, 191, 63], np.int32)
    pos_c = np.array([0, 10, -1, 9, 7], np.int32)
    for paged in (False, True):
        n_rows = B * max_pages * ps if paged else B * 10
        rows = np.full((n_rows, W), -7.0, dtype=np.float32)
        p = pos if paged else pos_c
        oracle.cache_append(x[:, :DL], x[:, DL:], "f32", p, rows, "f32",
                            page_size=ps if paged else 0, seq_stride=0 if paged else 10,
                            block_table=perm if paged else None)
        written = set()
        for b in range(B):
            t = int(p[b])
            cap = max_pages * ps if paged else 10
            if t < 0 or t >= cap:
                continue
            row = int(perm[b, t // ps]) * ps + t % ps if paged else b * 10 + t
            assert np.array_equal(rows[row], x[b])
            written.add(row)
        others = [i for i in range(n_rows) if i not in written]
        assert np.all(rows[others] == -7.0)
        assert len(written) == (4 if paged else 3)


def test_unmapped_page_is_skipped():
    """A negative block-table entry names no page (the convention the library
    and the oracle share: a caller that has not mapped a page yet marks it -1):
    the append of that sequence writes nothing, and the sequences after it are
    still written."""
    ps = 64
    bt = np.array([[0, 1], [-1, 2], [3, -1], [4, 5]], np.int32)
    pos = np.array([5, 3, 70, 64], np.int32)  # sequences 1 and 2 land on unmapped pages
    x = np.random.default_rng(10).standard_normal((4, W)).astype(np.float32)
    rows = np.full((6 * ps, W), -7.0, dtype=np.float32)
    oracle.cache_append(x[:, :DL], x[:, DL:], "f32", pos, rows, "f32", page_size=ps,
                        block_table=bt)
    assert np.array_equal(rows[0 * ps + 5], x[0])
    assert np.array_equal(rows[5 * ps + 0], x[3])
    others = [i for i in range(6 * ps) if i not in (5, 5 * ps)]
    assert np.all(rows[others] == -7.0)

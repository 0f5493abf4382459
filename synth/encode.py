"""Packing of drawn values into the stored formats.

These routines only produce the bits that are handed to both the kernels and
the oracle; each of those decodes the bits on its own.

* bf16: the upper half of an IEEE-754 binary32, rounded to nearest even.
* e4m3: the OCP 8-bit floating point format E4M3 ("FN" variant: exponent bias
  7, no infinities, S.1111.111 is NaN, largest finite 448).  Rows are scaled
  by one fp32 factor so that the largest magnitude maps to 448, then rounded
  to nearest even and saturated to +-448.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
_TINY = np.float32(2.0 ** -126)


def round_to_f32(x: np.ndarray) -> np.ndarray:
    """Round doubles to binary32 (round to nearest even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """binary32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> binary32 values (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _e4m3_encode(y: np.ndarray) -> np.ndarray:
    """binary32 values with |y| <= 448 -> E4M3 codes, round to nearest even."""
    y = np.ascontiguousarray(y, dtype=np.float32)
    sign = (y.view(np.uint32) >> np.uint32(31)).astype(np.uint8)
    a = np.abs(y)
    code = np.zeros(a.shape, dtype=np.uint8)
    sub = a < np.float32(2.0 ** -6)
    # subnormal range: spacing 2^-9, scaling by 2^9 is exact, rint is ties-to-even
    code[sub] = np.rint(a[sub] * np.float32(512.0)).astype(np.uint8)
    nrm = ~sub
    bits = a[nrm].view(np.uint32)
    lsb = (bits >> np.uint32(20)) & np.uint32(1)
    bits = (bits + np.uint32(0x7FFFF) + lsb) & np.uint32(0xFFF00000)
    exp = (bits >> np.uint32(23)).astype(np.int32) - 127 + 7
    man = ((bits >> np.uint32(20)) & np.uint32(7)).astype(np.int32)
    code[nrm] = ((exp << 3) | man).astype(np.uint8)
    return code | (sign << np.uint8(7))


def quantize_rows_e4m3(rows: np.ndarray):
    """Per-row scaled E4M3 quantization of a float32 [n, w] array.

    scale = max(amax, 2^-126) / 448 in fp32; code = RNE(x / scale) saturated
    to +-448.  Returns (codes uint8 [n, w], scale float32 [n]).
    """
    rows = np.ascontiguousarray(rows, dtype=np.float32)
    amax = np.max(np.abs(rows), axis=1)
    scale = (np.maximum(amax, _TINY) / np.float32(E4M3_MAX)).astype(np.float32)
    y = rows / scale[:, None]
    y = np.clip(y, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    return _e4m3_encode(y), scale

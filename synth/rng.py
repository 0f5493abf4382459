"""Counter-based random numbers: SplitMix64 mixing + Box-Muller normals.

Every value is a pure function of (seed, stream id, element index), so any
sub-range of a tensor can be regenerated on its own (the tests recompute single
sequences of a large cache this way) and the result never depends on how the
work is chunked or threaded.

SplitMix64 is the generator of Steele, Lea and Flood, "Fast splittable
pseudorandom number generators" (OOPSLA 2014): state_i = seed + (i+1)*gamma with
gamma = 0x9E3779B97F4A7C15, output = mix(state_i).  Normals use the Box-Muller
transform (Box and Muller, 1958) on pairs of 53-bit uniforms.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_MASK64 = (1 << 64) - 1
_CHUNK = 1 << 19  # elements per worker task


def _mix(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def _mix_int(z: int) -> int:
    z &= _MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
    return z ^ (z >> 31)


def stream_seed(seed: int, stream: int) -> int:
    """64-bit key of one named stream (one tensor) under a base seed."""
    return _mix_int((int(seed) << 8) + int(stream))


def _workers() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def _chunked(fn, start: int, count: int, dtype) -> np.ndarray:
    """Evaluate fn(start_i, count_i) over chunks, in parallel threads (numpy
    releases the GIL inside its loops).  The result is identical to one call."""
    out = np.empty(count, dtype=dtype)
    if count <= _CHUNK:
        out[:] = fn(start, count)
        return out
    spans = [(o, min(_CHUNK, count - o)) for o in range(0, count, _CHUNK)]

    def run(span):
        o, n = span
        out[o:o + n] = fn(start + o, n)

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(run, spans))
    return out


def splitmix64_bits(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    """Raw 64-bit outputs for counters start .. start+count-1 (uint64)."""
    key = np.uint64(stream_seed(seed, stream))

    def fn(s, n):
        idx = np.arange(s + 1, s + 1 + n, dtype=np.uint64)
        return _mix(key + idx * _GAMMA)

    return _chunked(fn, start, count, np.uint64)


def uniform01(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    """Uniform doubles in [0, 1) from the top 53 bits (float64)."""
    key = np.uint64(stream_seed(seed, stream))

    def fn(s, n):
        idx = np.arange(s + 1, s + 1 + n, dtype=np.uint64)
        z = _mix(key + idx * _GAMMA)
        return (z >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)

    return _chunked(fn, start, count, np.float64)


def standard_normal(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    """N(0,1) doubles for elements start .. start+count-1 of a stream.

    Element 2j and 2j+1 come from one Box-Muller pair built from counters 2j
    (radius, u1 in (0,1]) and 2j+1 (angle, u2 in [0,1)): the even element is
    r*cos(2*pi*u2), the odd one r*sin(2*pi*u2).
    """
    key = np.uint64(stream_seed(seed, stream))

    def fn(s, n):
        p0 = s // 2
        p1 = (s + n + 1) // 2
        j = np.arange(p0, p1, dtype=np.uint64)
        z1 = _mix(key + (np.uint64(2) * j + np.uint64(1)) * _GAMMA)
        z2 = _mix(key + (np.uint64(2) * j + np.uint64(2)) * _GAMMA)
        u1 = ((z1 >> np.uint64(11)).astype(np.float64) + 1.0) * (1.0 / 9007199254740992.0)
        u2 = (z2 >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)
        r = np.sqrt(-2.0 * np.log(u1))
        th = 2.0 * np.pi * u2
        pair = np.empty((p1 - p0, 2), dtype=np.float64)
        pair[:, 0] = r * np.cos(th)
        pair[:, 1] = r * np.sin(th)
        flat = pair.reshape(-1)
        off = s - 2 * p0
        return flat[off:off + n]

    return _chunked(fn, start, count, np.float64)


def randint_uniform(seed: int, stream: int, lo: int, hi: int, count: int) -> np.ndarray:
    """Integers uniform on [lo, hi] inclusive (int64)."""
    u = uniform01(seed, stream, 0, count)
    return lo + np.floor(u * (hi - lo + 1)).astype(np.int64)


def permutation(seed: int, stream: int, n: int) -> np.ndarray:
    """Fisher-Yates shuffle of 0..n-1 driven by the stream (int64)."""
    perm = np.arange(n, dtype=np.int64)
    if n < 2:
        return perm
    u = uniform01(seed, stream, 0, n)
    for i in range(n - 1, 0, -1):
        j = int(u[i] * (i + 1))
        perm[i], perm[j] = perm[j], perm[i]
    return perm

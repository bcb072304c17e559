"""Independent brute-force views used to pin the oracle.

Nothing here shares code with the oracle: positions come from walking the
batch sequence by sequence (not from searching the offsets), cache rows are
found by numpy indexing of the pool's logical shape (not by stride
arithmetic), and rotations use Python's complex multiplication.
"""
from __future__ import annotations

import math

import numpy as np

from synth import cases as sc


def walk_tokens(case):
    """Yield (t, b, cache_seq, pos) by construction: sequence b's tokens are
    rows off_b .. off_b + len_b - 1, at positions cache_len + 0, 1, ..."""
    t = 0
    for b, n in enumerate(case.lengths):
        cseq = b + case.batch_offset
        for local in range(int(n)):
            yield t, b, cseq, int(case.caches[0].cache_lengths[cseq]) + local
            t += 1


def page_slot(cache, cseq: int, pos: int):
    return int(cache.lookup_table[cseq, pos // cache.page_size]), pos % cache.page_size


def as_f64(bits, dtype):
    return sc.bits_to_f64(np.asarray(bits), dtype)


def rope_complex(x: np.ndarray, freqs_row: np.ndarray, rope_dim: int, interleaved: bool):
    """Rotate pairs by Python complex multiplication; returns (values, pair_norms)."""
    y = [float(v) for v in x]
    mag = [abs(float(v)) for v in x]
    half = rope_dim // 2
    for i in range(half):
        j0, j1 = (2 * i, 2 * i + 1) if interleaved else (i, i + half)
        z = complex(float(x[j0]), float(x[j1])) * complex(float(freqs_row[2 * i]),
                                                          float(freqs_row[2 * i + 1]))
        y[j0], y[j1] = z.real, z.imag
        mag[j0] = mag[j1] = abs(z)
    return np.array(y), np.array(mag)


def bf16_table():
    """All finite bf16 values (as doubles) with their bits, sorted by value."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = sc.bits_to_f64(bits, sc.BF16)
    fin = np.isfinite(vals)
    bits, vals = bits[fin], vals[fin]
    # keep +0 only (-0 compares equal); sort by value
    keep = ~((vals == 0) & (bits == 0x8000))
    bits, vals = bits[keep], vals[keep]
    order = np.argsort(vals, kind="stable")
    return vals[order], bits[order]


def nearest_even_bf16(x: float, vals: np.ndarray, bits: np.ndarray) -> int:
    """bf16 bits of x by exhaustive neighbour search; ties go to the even
    significand; beyond the largest finite value by half an ulp -> inf."""
    if math.isnan(x):
        raise ValueError("nan")
    big = float(vals[-1])                        # largest finite bf16
    half_ulp_top = 2.0 ** (127 - 8)
    if x >= big + half_ulp_top:
        return 0x7F80
    if x <= -(big + half_ulp_top):
        return 0xFF80
    if x == 0.0:
        return 0x8000 if math.copysign(1.0, x) < 0 else 0x0000
    k = int(np.searchsorted(vals, x))
    cands = [i for i in (k - 1, k) if 0 <= i < len(vals)]
    best = min(cands, key=lambda i: (abs(float(vals[i]) - x), int(bits[i]) & 1))
    out = int(bits[best])
    if out == 0 and x < 0:
        out = 0x8000
    return out


def ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |x| (2^-133 below the normal range)."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    e = np.floor(np.log2(ax))
    return np.power(2.0, e - 7)


def ulp_f16(x: np.ndarray) -> np.ndarray:
    """Spacing of IEEE binary16 values at |x| (2^-24 below the normal range)."""
    ax = np.maximum(np.abs(x), 2.0 ** -14)
    e = np.floor(np.log2(ax))
    return np.power(2.0, e - 10)

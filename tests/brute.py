"""Independent brute-force views used to pin the oracle.

Nothing here shares code with the oracle: positions come from walking the
batch sequence by sequence (not from searching the offsets), cache rows are
found by numpy indexing of the pool's logical shape (not by stride
arithmetic), and rotations use Python's complex multiplication.
"""
from __future__ import annotations

import functools
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



def e4m3_table():
    """Every finite OCP E4M3 code (positive and negative) with its value,
    decoded from the bit fields: sign, exponent field e (bias 7), fraction m;
    e = 0 holds m * 2^-9."""
    codes, vals = [], []
    for c in range(256):
        sign, e, m = c >> 7, (c >> 3) & 0xF, c & 7
        if e == 15 and m == 7:
            continue                                  # NaN
        v = m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
        codes.append(c)
        vals.append(-v if sign else v)
    return np.array(codes, dtype=np.uint8), np.array(vals)


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    table = np.full(256, np.nan)
    c, v = e4m3_table()
    table[c] = v
    return table[np.asarray(codes, dtype=np.uint8)]


def nearest_even_e4m3(x: float) -> int:
    """Code of x by neighbour search among the non-negative finite values;
    ties go to the even code; magnitudes past 448 saturate."""
    c, v = e4m3_table()
    pos = v >= 0
    c, v = c[pos & ~((c == 0x80))], v[pos & ~((c == 0x80))]
    order = np.argsort(v)
    c, v = c[order], v[order]
    a = abs(x)
    if a >= 448.0:
        best = 0x7E
    else:
        k = int(np.searchsorted(v, a))
        cands = [i for i in (k - 1, k) if 0 <= i < len(v)]
        best = int(c[min(cands, key=lambda i: (abs(float(v[i]) - a), int(c[i]) & 1))])
    if math.copysign(1.0, x) < 0:
        best |= 0x80
    return best


def quantize_row_f32(values: np.ndarray, scale_dtype: str):
    """The row quantization in numpy binary32 arithmetic, codes by neighbour
    search: returns (codes uint8 [D], scale bits)."""
    v = np.asarray(values, dtype=np.float64).astype(np.float32)
    amax = np.max(np.abs(v)) if v.size else np.float32(0)
    s = np.float32(amax) / np.float32(448.0)
    if scale_dtype == sc.BF16:
        s = sc.bits_to_f64(sc.to_bits(np.array([s], np.float64), sc.BF16), sc.BF16).astype(
            np.float32)[0]
    r = np.float32(1.0) / s if s > 0 else np.float32(0.0)
    q = np.clip(v * r, np.float32(-448.0), np.float32(448.0))
    codes = np.array([nearest_even_e4m3(float(x)) for x in q], dtype=np.uint8)
    bits = sc.to_bits(np.array([float(s)]), scale_dtype)[0]
    return codes, bits


def ulp_e4m3(x: np.ndarray) -> np.ndarray:
    """Spacing of E4M3 values at |x| (2^-9 below the normal range)."""
    ax = np.maximum(np.abs(x), 2.0 ** -6)
    e = np.floor(np.log2(ax))
    return np.power(2.0, e - 3)


def f16_table():
    """All finite IEEE binary16 values (as doubles) with their bits, sorted by value."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16).astype(np.float64)
    fin = np.isfinite(vals)
    bits, vals = bits[fin], vals[fin]
    keep = ~((vals == 0) & (bits == 0x8000))
    bits, vals = bits[keep], vals[keep]
    order = np.argsort(vals, kind="stable")
    return vals[order], bits[order]


@functools.lru_cache(maxsize=None)
def _table_16(dtype: str):
    return bf16_table() if dtype == sc.BF16 else f16_table()


def round_exact_16(q, dtype: str):
    """Nearest-even bf16 / binary16 bits of an exact rational ``q``
    (fractions.Fraction) by neighbour search over every finite value of the
    type, with exact comparisons; also returns q's distance to the nearest
    rounding midpoint, relative to |q|.  Finite results only."""
    from fractions import Fraction
    vals, bits = _table_16(dtype)
    k = int(np.searchsorted(vals, float(q)))
    cands = [i for i in range(k - 2, k + 2) if 0 <= i < len(vals)]
    dist = {i: abs(Fraction(float(vals[i])) - q) for i in cands}
    best = min(cands, key=lambda i: (dist[i], int(bits[i]) & 1))
    lo = max((i for i in cands if Fraction(float(vals[i])) <= q), default=None)
    hi = min((i for i in cands if Fraction(float(vals[i])) > q), default=None)
    rel = Fraction(1)
    if lo is not None and hi is not None and q != 0:
        mid = (Fraction(float(vals[lo])) + Fraction(float(vals[hi]))) / 2
        rel = abs(q - mid) / abs(q)
    out = int(bits[best])
    if out == 0 and q < 0:
        out = 0x8000
    return out, rel

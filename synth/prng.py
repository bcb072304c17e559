"""Seeded pseudo-random streams for the synthetic inputs.

Integer draws (lengths, cache lengths, page permutations, special-value
positions) are counter-based: every draw is ``mix(key + (i + 1) * GOLDEN)`` for counter ``i``, where ``mix``
is the splitmix64 finaliser (Steele, Lea and Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014) and ``key`` is derived from the
case seed and a per-array stream number.  Draws are therefore independent of
the order in which arrays are generated and can be vectorised.

This module holds no arithmetic of the RoPE / paged-store method.
"""
from __future__ import annotations

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def _mix(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        return z ^ (z >> np.uint64(31))


def stream_key(seed: int, stream: int) -> np.uint64:
    """Key of stream ``stream`` of case seed ``seed``."""
    base = np.array([(seed & 0xFFFFFFFF) | ((stream & 0xFFFFFFFF) << 32)], dtype=np.uint64)
    return _mix(base)[0]


def raw(seed: int, stream: int, n: int, start: int = 0) -> np.ndarray:
    """``n`` 64-bit draws of a stream, counters ``start .. start+n-1``."""
    key = stream_key(seed, stream)
    ctr = np.arange(start + 1, start + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix(key + ctr * GOLDEN)


def uniform01(seed: int, stream: int, n: int, start: int = 0) -> np.ndarray:
    """Doubles in (0, 1] from the top 53 bits of each draw."""
    r = raw(seed, stream, n, start)
    return ((r >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)


def integers(seed: int, stream: int, n: int, lo: int, hi: int) -> np.ndarray:
    """Uniform integers in [lo, hi] (inclusive) as int64."""
    span = np.uint64(hi - lo + 1)
    return (raw(seed, stream, n) % span).astype(np.int64) + lo


def normal(seed: int, stream: int, n: int, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    """N(mean, std^2) doubles.

    Bulk normals come from numpy's PCG64 generator (O'Neill, "PCG: a family
    of simple fast space-efficient statistically good algorithms", 2014) with
    its ziggurat sampler, keyed by SeedSequence([seed, stream]); tens of
    millions of values per case make a pure splitmix64 + Box-Muller path
    too slow for the test-suite."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed & 0xFFFFFFFF,
                                                                    stream & 0xFFFFFFFF])))
    return g.standard_normal(n) * std + mean


def permutation(seed: int, stream: int, n: int) -> np.ndarray:
    """A permutation of 0..n-1 (argsort of random keys, stable)."""
    return np.argsort(raw(seed, stream, n), kind="stable").astype(np.int64)

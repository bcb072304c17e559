"""The GEMV parity bar (tests/gemv_parity.py) checked on the CPU: it accepts
the oracle's own outputs, and it rejects a plausible kernel mistake planted
in the oracle's exact results -- one term of every dot product dropped --
on a large share of the outputs."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from synth import cases as sc
from tests import brute
from tests import gemv_parity as gp


def _outputs(case, y):
    """Rounded normed and passed-through outputs of a given y (double)."""
    nn = case.n_normed
    g = brute.as_f64(case.gamma[:nn], case.dtype)
    r = 1.0 / np.sqrt((y[:, :nn] ** 2).mean(axis=1) + float(np.float32(case.epsilon)))
    normed = sc.to_bits(y[:, :nn] * r[:, None] * g[None, :], case.dtype)
    unnormed = sc.to_bits(y[:, nn:], case.dtype)
    return normed, unnormed


@pytest.mark.parametrize("small", [True, False])
def test_bar_accepts_exact_and_rejects_a_dropped_term(small):
    case = sc.gemv_norm(small=small)
    res = oracle.run_gemv(case)
    nn, n = case.n_normed, case.n
    # the oracle's own outputs pass
    gp.check(case, res, res.normed, res.unnormed)
    # drop one term per column from the exact sums
    x = brute.as_f64(case.x[:, :case.k], case.dtype)
    w = brute.as_f64(case.w[:, :case.k], case.dtype)
    kk = np.random.default_rng(0).integers(0, case.k, n)
    y_bad = res.y_exact - x[:, kk] * w[np.arange(n), kk][None, :]
    normed, unnormed = _outputs(case, y_bad)
    nt, ut = gp.bounds(case, res)
    for bits, ora, tol, width in ((normed, res.normed, nt, nn), (unnormed, res.unnormed, ut, n - nn)):
        g = sc.bits_to_f64(bits, case.dtype)
        o = sc.bits_to_f64(ora[:, :width], case.dtype)
        allow = tol + gp.ulp(np.maximum(np.abs(g), np.abs(o)), case.dtype)
        assert np.mean(np.abs(g - o) > allow) > 0.2
    with pytest.raises(AssertionError):
        full_n = np.full((case.m, case.normed_row_stride), sc.SENTINEL[case.dtype], normed.dtype)
        full_u = np.full((case.m, case.unnormed_row_stride), sc.SENTINEL[case.dtype], normed.dtype)
        full_n[:, :nn], full_u[:, :n - nn] = normed, unnormed
        gp.check(case, res, full_n, full_u)

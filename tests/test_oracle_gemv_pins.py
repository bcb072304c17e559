"""Pins of the oracle's fused GEMV + partial RMSNorm (MatmulFusedPartialRMSNorm
page: Summary, execute, Args) against facts that do not come from the oracle.

* The GEMV: exact rational sums (Python fractions) on small inputs whose m,
  n, k and padded row strides all differ, so a transposed or mis-strided
  operand, a dropped term or a row mix-up shows; each passed-through output
  is the nearest-even rounding of the exact sum, found by search over every
  bf16 value or by numpy's float32 conversion.
* The partial norm: a closed form -- y = (3, 4 | 5, -7, 0.5) with epsilon
  0.5 gives normed outputs (3, 4) / sqrt(12.5 + 0.5) times gamma and
  passes 5, -7, 0.5 through exactly; unit mean square with gamma = 1 and
  epsilon = 0; the normed part is invariant under scaling x by a power of
  two while the rest scales exactly; weight_offset is not consumed.
* Output padding keeps its sentinels.
* W stored [k][n] (transpose_b False, the page's Parameters): exact rational
  sums indexed W[k][j] on a case whose k, n and padded stride all differ,
  a square case whose transpose differs (W != W^T), and bit equality with
  the [n][k] form on the same matrix.
"""
from __future__ import annotations

import fractions
import math

import numpy as np

import oracle
from synth import cases as sc
from tests import brute


def _exact(case):
    """y[i][j] as exact fractions, by direct summation over k (W read as
    w[j][k] when stored [n][k], as w[k][j] when stored [k][n])."""
    F = fractions.Fraction
    x = brute.as_f64(case.x[:, :case.k], case.dtype)
    if case.transpose_b:
        w = brute.as_f64(case.w[:, :case.k], case.dtype)
        wjk = lambda j, kk: w[j, kk]
    else:
        w = brute.as_f64(case.w[:, :case.n], case.dtype)
        wjk = lambda j, kk: w[kk, j]
    return [[sum(F(float(x[i, kk])) * F(float(wjk(j, kk))) for kk in range(case.k))
             for j in range(case.n)] for i in range(case.m)]


def _rounded_bits(v: float, dtype: str) -> int:
    if dtype == sc.F32:
        return int(np.float32(v).view(np.uint32))
    vals, bits = brute.bf16_table()
    return int(brute.nearest_even_bf16(v, vals, bits))


def _closed_form_case(dtype, eps=0.5, w_off=0.0):
    # x = e_0 (a unit in column 0) picks column 0 of W: y_j = W[j][0]
    case = sc.make_gemv_case("closed", 3, dtype, m=1, k=16, n=5, n_normed=2, epsilon=eps,
                             weight_offset=w_off)
    x = np.zeros((1, 16))
    x[0, 0] = 1.0
    case.x = sc.to_bits(x, dtype)
    w = np.zeros((5, 16))
    w[:, 0] = [3.0, 4.0, 5.0, -7.0, 0.5]
    w[:, 1:] = 0.0
    case.w = sc.to_bits(w, dtype)
    case.gamma = sc.to_bits(np.array([1.0, 2.0]), dtype)
    return case


def test_gemv_matches_exact_rational_sums():
    for dtype in (sc.BF16, sc.F32, sc.F16):
        case = sc.make_gemv_case("pin", 11, dtype, m=3, k=24, n=7, n_normed=0, x_pad=3,
                                 w_pad=5, out_pad=2)
        res = oracle.run_gemv(case)
        assert res.status == 0
        ex = _exact(case)
        for i in range(case.m):
            for j in range(case.n):
                y = float(ex[i][j])
                bound = 2.0 ** -50 * res.abs_dot[i, j] + 1e-300
                assert abs(res.y_exact[i, j] - y) <= bound, (dtype, i, j)
                if dtype != sc.F16:
                    assert int(res.unnormed[i, j]) == _rounded_bits(y, dtype), (dtype, i, j)
                else:
                    assert int(res.unnormed[i, j]) == int(np.float16(y).view(np.uint16))
        # abs_dot is sum_k |x_k w_jk|
        x = brute.as_f64(case.x[:, :case.k], case.dtype)
        w = brute.as_f64(case.w[:, :case.k], case.dtype)
        assert np.allclose(res.abs_dot, np.abs(x) @ np.abs(w).T, rtol=1e-14)


def test_nothing_normed_is_numpy_matmul():
    case = sc.make_gemv_case("pin", 12, sc.F32, m=2, k=64, n=40, n_normed=0)
    res = oracle.run_gemv(case)
    x = brute.as_f64(case.x, sc.F32)
    w = brute.as_f64(case.w, sc.F32)
    y = x @ w.T
    assert np.all(np.abs(res.y_exact - y) <= 1e-13 * (np.abs(x) @ np.abs(w).T))
    got = brute.as_f64(res.unnormed[:, :40], sc.F32)
    assert np.allclose(got, y, rtol=2.0 ** -23, atol=0)


def test_partial_norm_closed_form():
    for dtype in (sc.F32, sc.BF16):
        case = _closed_form_case(dtype)
        res = oracle.run_gemv(case)
        assert res.status == 0
        eps32 = float(np.float32(0.5))
        r = 1.0 / math.sqrt((9.0 + 16.0) / 2.0 + eps32)
        want = [3.0 * r * 1.0, 4.0 * r * 2.0]
        assert [int(b) for b in res.normed[0, :2]] == [_rounded_bits(v, dtype) for v in want]
        assert [int(b) for b in res.unnormed[0, :3]] == \
            [_rounded_bits(v, dtype) for v in (5.0, -7.0, 0.5)]
        assert res.r[0] == r


def test_partial_norm_unit_mean_square_and_scale_invariance():
    case = sc.make_gemv_case("pin", 13, sc.F32, m=2, k=32, n=24, n_normed=17, epsilon=0.0,
                             out_pad=3)
    case.gamma = sc.to_bits(np.ones(17), sc.F32)
    r1 = oracle.run_gemv(case)
    normed = brute.as_f64(r1.normed[:, :17], sc.F32)
    assert np.allclose((normed ** 2).mean(axis=1), 1.0, rtol=1e-6)
    # x -> 4x (exact): normed bits unchanged, passed-through values exactly 4x
    case.x = sc.to_bits(4.0 * brute.as_f64(case.x, sc.F32), sc.F32)
    r2 = oracle.run_gemv(case)
    assert np.array_equal(r1.normed, r2.normed)
    assert np.array_equal(brute.as_f64(r2.unnormed[:, :7], sc.F32),
                          4.0 * brute.as_f64(r1.unnormed[:, :7], sc.F32))
    # padding columns keep their sentinels
    assert np.all(r1.normed[:, 17:] == sc.SENTINEL[sc.F32])
    assert np.all(r1.unnormed[:, 7:] == sc.SENTINEL[sc.F32])


def test_weight_offset_is_not_consumed():
    a = oracle.run_gemv(_closed_form_case(sc.BF16, w_off=0.0))
    b = oracle.run_gemv(_closed_form_case(sc.BF16, w_off=0.5))
    assert np.array_equal(a.normed, b.normed) and np.array_equal(a.unnormed, b.unnormed)


def test_rows_are_independent():
    case = sc.make_gemv_case("pin", 14, sc.BF16, m=3, k=40, n=12, n_normed=5)
    full = oracle.run_gemv(case)
    for i in range(3):
        one = sc.make_gemv_case("pin", 14, sc.BF16, m=3, k=40, n=12, n_normed=5)
        one.m, one.x = 1, case.x[i:i + 1]
        r = oracle.run_gemv(one)
        assert np.array_equal(r.normed[0], full.normed[i])
        assert np.array_equal(r.unnormed[0], full.unnormed[i])


def test_w_stored_k_by_n_matches_exact_rational_sums():
    for dtype in (sc.BF16, sc.F32, sc.F16):
        case = sc.make_gemv_case("pin_t", 15, dtype, m=2, k=24, n=9, n_normed=0, x_pad=3,
                                 w_pad=7, out_pad=2, transpose_b=False)
        assert case.w.shape == (24, 16)
        res = oracle.run_gemv(case)
        assert res.status == 0
        ex = _exact(case)
        for i in range(case.m):
            for j in range(case.n):
                y = float(ex[i][j])
                assert abs(res.y_exact[i, j] - y) <= 2.0 ** -50 * res.abs_dot[i, j] + 1e-300
                if dtype == sc.F16:
                    assert int(res.unnormed[i, j]) == int(np.float16(y).view(np.uint16))
                else:
                    assert int(res.unnormed[i, j]) == _rounded_bits(y, dtype), (dtype, i, j)


def test_w_stored_k_by_n_is_not_read_as_n_by_k():
    # a square W whose transpose differs: reading W[j][k] in place of W[k][j]
    # gives other sums; x = e_1 picks row 1 of the stored [k][n] array
    case = sc.make_gemv_case("pin_t", 16, sc.F32, m=1, k=8, n=8, n_normed=0, transpose_b=False)
    stored = np.arange(64, dtype=np.float64).reshape(8, 8)   # stored[k][j]
    case.w = sc.to_bits(stored, sc.F32)
    x = np.zeros((1, 8))
    x[0, 1] = 1.0
    case.x = sc.to_bits(x, sc.F32)
    res = oracle.run_gemv(case)
    assert res.y_exact[0].tolist() == stored[1].tolist()     # y_j = W[k=1][j]


def test_w_stored_k_by_n_equals_w_stored_n_by_k():
    for dtype in (sc.BF16, sc.F32):
        a = sc.make_gemv_case("pin_t", 17, dtype, m=3, k=40, n=21, n_normed=13, w_pad=4)
        b = sc.make_gemv_case("pin_t", 17, dtype, m=3, k=40, n=21, n_normed=13, w_pad=4,
                              transpose_b=False)
        assert np.array_equal(a.w[:, :40].T, b.w[:, :21])
        ra, rb = oracle.run_gemv(a), oracle.run_gemv(b)
        assert np.array_equal(ra.normed, rb.normed) and np.array_equal(ra.unnormed, rb.unnormed)

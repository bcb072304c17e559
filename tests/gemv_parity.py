"""Parity bar of the fused GEMV + partial RMSNorm, derived from the kernel's
binary32 arithmetic (u = 2^-24).

The GEMV.  Each output y_j is the sum of k products.  One wave computes
it: each of its 64 lanes takes every 64th 16-byte chunk, which the lane
adds in k order (n_l = ceil(kc / 64) * E terms, E elements per chunk) --
one fused multiply-add per term for fp32, one packed dot product per pair
of terms for bf16 and f16 (their products are exact in binary32, so it
rounds at most once per term) -- and then adds the 64 partial sums in a
6-level tree.  Recursive summation of n terms errs by at most
gamma_n = n u / (1 - n u) times the sum of the terms' magnitudes, so
    |y^ - y| <= D_j = gamma_{n_l + 6} * A_j,    A_j = sum_k |x_k w_jk|,
with y the oracle's exact sum.  With W stored [k][n] (transpose_b = 0) k
is cut into S <= ceil(k / 512) slices; in each, a thread adds the terms of
8 consecutive rows of every 512 in k order, one fused multiply-add per term
(n_l <= 8 ceil(k / 512)), then come the 3-level butterfly over the wave's
row groups, the eight wave sums (7 adds) and the S slice sums (S - 1 adds):
D_j = gamma_{n_l + S + 9} * A_j.  A passed-through output
is y^ rounded to the dtype, the oracle's is y rounded: they differ by at
most D_j plus one ulp of the larger.

The norm.  The kernel squares and sums the binary32 y^ values with 256
threads: n_2 = ceil(n_normed / 256) fused multiply-adds per thread, the
6-level tree in each of four waves, then the four wave sums (3 adds):
    |s^ - S| <= E_S = gamma_{n_2 + 9} (S + D_S) + D_S,
    S = sum y_j^2,  D_S = sum (2 |y_j| D_j + D_j^2).
M = S / n_normed + eps takes two roundings (the division, the add), so
    |M^ - M| <= E_M = E_S / n_normed + 2u (M + E_S / n_normed),
and r = 1 / sqrt(M) takes the square root (within one ulp, 2u) and the
reciprocal (u):  rho_r = 0.5 E_M / (M - E_M) + 3u  bounds r^'s relative
error.  out_j = (y_j r) gamma_j takes two more roundings (2u), so
    |out^ - out| <= |gamma_j| r D_j (1 + rho_r) + |out| (rho_r + 2u) (1 + 4u),
and the stored values differ by at most that plus one ulp of the larger.
Every bound is applied with a 1 % margin for the second-order terms.
"""
from __future__ import annotations

import numpy as np

from synth import cases as sc
from tests import brute

U = 2.0 ** -24


def _gamma(n) -> float:
    return n * U / (1.0 - n * U)


def ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == sc.BF16:
        return brute.ulp_bf16(x)
    if dtype == sc.F16:
        return brute.ulp_f16(x)
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return np.power(2.0, np.floor(np.log2(ax)) - 23)


def bounds(case, res):
    """(normed_tol [m, n_normed], unnormed_tol [m, n - n_normed]) before the
    final one-ulp allowance, from the oracle's exact y, sum |x w| and r."""
    E = 4 if case.dtype == sc.F32 else 8
    kc = case.k // E
    if getattr(case, "transpose_b", 1):
        D = _gamma(-(-kc // 64) * E + 6) * res.abs_dot       # [m, n]
    else:
        rounds = -(-case.k // 512)
        D = _gamma(8 * rounds + rounds + 9) * res.abs_dot
    nn = case.n_normed
    un_tol = 1.01 * D[:, nn:]
    if nn == 0:
        return np.zeros((case.m, 0)), un_tol
    y = res.y_exact[:, :nn]
    Dn = D[:, :nn]
    S = np.sum(y * y, axis=1)
    DS = np.sum(2.0 * np.abs(y) * Dn + Dn * Dn, axis=1)
    n2 = -(-nn // 256)
    ES = _gamma(n2 + 9) * (S + DS) + DS
    M = S / nn + float(np.float32(case.epsilon))
    EM = ES / nn + 2.0 * U * (M + ES / nn)
    rho = 0.5 * EM / np.maximum(M - EM, 1e-300) + 3.0 * U
    g = np.abs(sc.bits_to_f64(case.gamma[:nn], case.dtype))
    r = res.r[:, None]
    out = np.abs(y) * r * g[None, :]
    nt = g[None, :] * r * Dn * (1.0 + rho[:, None]) + out * (rho[:, None] + 2.0 * U) * (1 + 4 * U)
    return 1.01 * nt, un_tol


def check(case, res, normed_bits: np.ndarray, unnormed_bits: np.ndarray) -> dict:
    """Assert the GPU outputs against the oracle's; padding keeps its sentinels."""
    nn, n, dt = case.n_normed, case.n, case.dtype
    nt, ut = bounds(case, res)
    rep = {}
    for name, gpu, ora, tol, width, stride in (
            ("normed", normed_bits, res.normed, nt, nn, case.normed_row_stride),
            ("unnormed", unnormed_bits, res.unnormed, ut, n - nn, case.unnormed_row_stride)):
        if width == 0:
            continue
        g = sc.bits_to_f64(gpu[:, :width], dt)
        o = sc.bits_to_f64(ora[:, :width], dt)
        allow = tol + ulp(np.maximum(np.abs(g), np.abs(o)), dt)
        err = np.abs(g - o)
        bad = ~(err <= allow)
        if bad.any():
            i, j = np.argwhere(bad)[0]
            raise AssertionError(f"{case.name} {name}[{i},{j}]: gpu {g[i, j]!r} oracle {o[i, j]!r} "
                                 f"allowed {allow[i, j]!r} ({int(bad.sum())} bad)")
        assert np.all(gpu[:, width:stride] == sc.SENTINEL[dt]), f"{name}: padding written"
        rep[f"{name}_exact_rate"] = float(np.mean(gpu[:, :width] == ora[:, :width]))
        rep[f"{name}_max_err_over_allowed"] = float(np.max(err / allow))
    return rep

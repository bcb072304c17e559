"""Pins of the oracle's RMSNorm branches and of the dual band's own parts.

* multiply_before_cast = false (fused_dual_qk_rms_norm_rope_ragged_paged
  page, Signature: the flag is named there, nothing more): the reading is
  n = dtype(x r), g' = dtype(gamma + w), m = dtype(n g'), then the rotation
  and one final rounding.  The closed form here computes r exactly (decimal
  arithmetic to 60 digits), every product and sum as an exact rational, and
  every rounding by neighbour search over all values of the type -- nothing
  from the oracle.  At position 0 the output is m itself; at a later
  position each pair is the exact rotation of (m_j0, m_j1) by the table's
  binary32 (cos, sin), rounded once.
* The dual band (same page, Description: each row selects its band's cache,
  gamma, epsilon and output; the index band's cache is a single-head K-only
  cache): a brute-force walk of both bands with caches of different page
  sizes and cache lengths and different epsilons, the index cache with one
  plane; rotations by Python complex multiplication, rows found by indexing
  the pools' logical shapes.
* The GPU parity bar for multiply_before_cast = false tells the flag's two
  values apart: fed the oracle's multiply_before_cast = true output, it
  fails; fed the false output, it passes.
"""
from __future__ import annotations

import decimal
from fractions import Fraction

import numpy as np
import pytest

import oracle
from synth import cases as sc
from tests import brute

decimal.getcontext().prec = 60

# distance (relative) from a rounding midpoint that the oracle's double
# evaluation of x r or of a rotation cannot cross (a few 2^-53)
SAFE = Fraction(1, 2 ** 40)


def _exact_r(x: np.ndarray, eps: float) -> decimal.Decimal:
    """1 / sqrt(mean(x^2) + eps) to 60 digits, x and eps exact binary values."""
    ss = sum(Fraction(float(v)) ** 2 for v in x)
    ms = ss / len(x) + Fraction(float(np.float32(eps)))
    d = decimal.Decimal(ms.numerator) / decimal.Decimal(ms.denominator)
    return 1 / d.sqrt()


def _frac(d: decimal.Decimal) -> Fraction:
    return Fraction(d)


def _mbc_false_head(x, gamma, w, eps, dtype):
    """m_j = dtype(dtype(x_j r) * dtype(gamma_j + w)) by exact arithmetic;
    also the single-rounding value x_j r (gamma_j + w) for the true branch.
    Every rounding is checked to sit clear of its midpoint."""
    r = _exact_r(x, eps)
    m, true_vals = [], []
    for xj, gj in zip(x, gamma):
        xr = _frac(decimal.Decimal(float(xj)) * r)
        n_bits, rel = brute.round_exact_16(xr, dtype)
        assert rel > SAFE, "choose inputs away from a midpoint of the first rounding"
        n = Fraction(float(sc.bits_to_f64(np.array([n_bits], np.uint16), dtype)[0]))
        g_bits, rel_g = brute.round_exact_16(Fraction(float(gj)) + Fraction(float(w)), dtype)
        g = Fraction(float(sc.bits_to_f64(np.array([g_bits], np.uint16), dtype)[0]))
        m_bits, rel_m = brute.round_exact_16(n * g, dtype)
        m.append(Fraction(float(sc.bits_to_f64(np.array([m_bits], np.uint16), dtype)[0])))
        true_vals.append(xr * (Fraction(float(gj)) + Fraction(float(w))))
    return m, true_vals


def _rotate_exact(m, freqs_row, R, interleaved, dtype):
    """Rounded bits of the exact rotation of the leading R dims of m (the
    rest pass as m), with each result's distance from its midpoint."""
    out = list(m)
    half = R // 2
    for i in range(half):
        j0, j1 = (2 * i, 2 * i + 1) if interleaved else (i, i + half)
        c, s = Fraction(float(freqs_row[2 * i])), Fraction(float(freqs_row[2 * i + 1]))
        out[j0], out[j1] = m[j0] * c - m[j1] * s, m[j0] * s + m[j1] * c
    res = [brute.round_exact_16(v, dtype) for v in out]
    return np.array([b for b, _ in res], np.uint16), [rel for _, rel in res]


def _mbc_case(dtype, interleaved, w=0.5, eps=0.6875):
    # one token at position 0 (sequence 0) and one at position 5 (sequence 1);
    # Q and K from the buffer; head_dim 64, full rope
    D = 64
    case = sc.make_norm_case("pin_mbc0", 61, dtype, [1, 1], [0, 5], Hq=2, Hk=1, D=D, rope_dim=D,
                             interleaved=interleaved, theta=1e4, max_seq_len=16, P=8, L=1,
                             layer=0, k_in_cache=False, eps=eps, weight_offset=w,
                             multiply_before_cast=False)
    # x: a fixed ramp of exact 16-bit values (different per head); gammas in
    # [0.5, 1) with the last bit of the type set (spacing sp there), so that
    # gamma + 0.5 lands halfway between two values of [1, 2) and rounds
    j = np.arange(D)
    sp = 2.0 ** -8 if dtype == sc.BF16 else 2.0 ** -11
    heads = []
    for h in range(4):                       # 2 Q, 1 K, 1 V
        heads.append((1.0 + (j + 7 * h) % 29 / 32.0) * np.where((j + h) % 3 == 0, -1.0, 1.0))
    row = np.concatenate(heads)
    case.buf[:] = sc.to_bits(np.tile(row, (2, 1)), dtype)
    gq = 0.5 + (2 * j + 1) * sp
    gk = 0.5 + (2 * ((j + 17) % D) + 1) * sp
    case.bands[0].q_gamma = sc.to_bits(gq, dtype)
    case.bands[0].k_gamma = sc.to_bits(gk, dtype)
    return case


@pytest.mark.parametrize("dtype", [sc.BF16, sc.F16])
@pytest.mark.parametrize("interleaved", [True, False])
def test_multiply_after_cast_closed_form(dtype, interleaved):
    case = _mbc_case(dtype, interleaved)
    res = oracle.run_case(case)
    assert res.status == 0
    cache = case.caches[0]
    D, Hq = 64, 2
    w = float(sc.bits_to_f64(sc.to_bits(np.array([case.weight_offset]), dtype), dtype)[0])
    n_diff_true = 0
    for t, pos in ((0, 0), (1, 5)):
        cseq = t
        page, slot = brute.page_slot(cache, cseq, pos)
        for h in range(Hq + 1):
            x = brute.as_f64(case.buf[t, h * D:(h + 1) * D], dtype)
            gbits = case.bands[0].q_gamma if h < Hq else case.bands[0].k_gamma
            g = brute.as_f64(gbits, dtype)
            m, true_vals = _mbc_false_head(x, g, w, case.bands[0].epsilon, dtype)
            want, rels = _rotate_exact(m, case.freqs[pos], D, interleaved, dtype)
            assert min(rels) > SAFE, "choose inputs away from a midpoint of the final rounding"
            got = (res.q_out[0][t, h * D:(h + 1) * D] if h < Hq
                   else res.pools[0][page, 0, 0, slot, 0])
            assert np.array_equal(got, want), (t, h, np.flatnonzero(got != want)[:8])
            if pos == 0:
                # the one-rounding value differs: the closed form can tell the branches apart
                t_bits = np.array([brute.round_exact_16(v, dtype)[0] for v in true_vals], np.uint16)
                n_diff_true += int((t_bits != want).sum())
    assert n_diff_true >= 8, "the inputs do not separate the two readings"


@pytest.mark.parametrize("dtype", [sc.BF16, sc.F16])
def test_multiply_before_cast_true_rounds_once(dtype):
    # with the flag on, the same inputs give one rounding of the exact
    # x r (gamma + w) at position 0
    case = _mbc_case(dtype, True)
    case.multiply_before_cast = True
    res = oracle.run_case(case)
    D = 64
    w = float(sc.bits_to_f64(sc.to_bits(np.array([case.weight_offset]), dtype), dtype)[0])
    x = brute.as_f64(case.buf[0, :D], dtype)
    g = brute.as_f64(case.bands[0].q_gamma, dtype)
    _, true_vals = _mbc_false_head(x, g, w, case.bands[0].epsilon, dtype)
    want = np.array([brute.round_exact_16(v, dtype)[0] for v in true_vals], np.uint16)
    assert np.array_equal(res.q_out[0][0, :D], want)


# --------------------------------------------------------------------------
# the dual band's own parts
# --------------------------------------------------------------------------

def _norm_rope(x, gamma, w, eps, pos_row, R, interleaved):
    """Double-precision norm (mean square over the head, eps inside the
    root, gamma + w) then complex rotation of the leading R dims."""
    y = x / np.sqrt(np.mean(x * x) + float(np.float32(eps))) * (gamma + w)
    return brute.rope_complex(y, pos_row, R, interleaved)


@pytest.mark.parametrize("dtype", [sc.F32, sc.BF16])
@pytest.mark.parametrize("interleaved", [True, False])
def test_dual_band_brute_force(dtype, interleaved):
    lens = [4, 0, 7, 2]
    cl_main = [3, 11, 0, 17]
    cl_index = [9, 0, 21, 1]
    R, D = 32, 64
    case = sc.make_dual_case("pin_dual", 62, dtype, lens, Hq_main=4, Hk_main=2, Hq_index=2, D=D,
                             rope_dim=R, interleaved=interleaved, theta=1e4, max_seq_len=64,
                             P_main=8, P_index=4, eps_main=1e-6, eps_index=0.25,
                             weight_offset=0.125, cache_lengths=cl_main,
                             index_cache_lengths=cl_index)
    main, index = case.caches
    assert index.kv_planes == 1 and index.num_kv_heads == 1 and main.kv_planes == 2
    before = [c.materialize() for c in case.caches]
    res = oracle.run_case(case)
    assert res.status == 0
    w = float(sc.bits_to_f64(sc.to_bits(np.array([0.125]), dtype), dtype)[0])
    tol = 2.0 ** -22 if dtype == sc.F32 else 2.0 ** -7
    bands = case.bands
    written = [set(), set()]
    t = 0
    for b, n in enumerate(lens):
        for local in range(n):
            for bi, band in enumerate(bands):
                cache = case.caches[band.cache]
                cl = cl_main if bi == 0 else cl_index
                pos = cl[b] + local
                page, slot = brute.page_slot(cache, b, pos)
                frow = case.freqs[pos]
                gq = brute.as_f64(band.q_gamma, dtype)
                gk = brute.as_f64(band.k_gamma, dtype)
                for h in range(band.n_q_heads):
                    x = brute.as_f64(case.buf[t, band.q_col + h * D:band.q_col + (h + 1) * D],
                                     dtype)
                    y, mag = _norm_rope(x, gq, w, band.epsilon, frow, R, interleaved)
                    got = brute.as_f64(res.q_out[bi][t, h * D:(h + 1) * D], dtype)
                    assert np.all(np.abs(got - y) <= tol * np.maximum(mag, np.abs(y))), \
                        (bi, t, h)
                for h in range(cache.num_kv_heads):
                    x = brute.as_f64(before[band.cache][page, 0, 0, slot, h], dtype)
                    y, mag = _norm_rope(x, gk, w, band.epsilon, frow, R, interleaved)
                    got = brute.as_f64(res.pools[band.cache][page, 0, 0, slot, h], dtype)
                    assert np.all(np.abs(got - y) <= tol * np.maximum(mag, np.abs(y))), \
                        (bi, "k", t, h)
                    written[band.cache].add((page, 0, 0, slot, h))
            t += 1
    # nothing else in either pool moved
    for ci in range(2):
        mask = np.ones(before[ci].shape[:5], dtype=bool)
        for wr in written[ci]:
            mask[wr] = False
        assert np.array_equal(res.pools[ci][mask], before[ci][mask]), ci
    # Q outputs have exactly the band's width
    assert res.q_out[1].shape == (case.T, 2 * D)


# --------------------------------------------------------------------------
# the GPU bar tells multiply_before_cast's values apart
# --------------------------------------------------------------------------

def _flag_case(dtype):
    # the shape of the GPU test of multiply_before_cast = false
    return sc.make_norm_case("norm_mbc0", 16, dtype, [25, 9], [0, 31], Hq=6, Hk=2, D=128,
                             rope_dim=64, interleaved=True, theta=1e4, max_seq_len=512, P=32,
                             L=2, layer=1, k_in_cache=False, multiply_before_cast=False,
                             weight_offset=0.5)


def _check_q(case, got_rows, res, parity):
    D, Hq = 128, 6
    tr = res.traces[0]
    rep = parity.Report()
    wide = parity.flip_mask(tr["q_pre"].reshape(-1, D), case.dtype, D, case.rope_dim,
                            case.interleaved, case.rope_tail)
    parity.check_rows(got_rows.reshape(-1, D), res.q_out[0].reshape(-1, D),
                      tr["q_exact"].reshape(-1, D), tr["q_mag"].reshape(-1, D),
                      np.zeros(D, bool), case.dtype, 1, "q", rep, wide=wide,
                      min_exact=parity.MBC_OFF_MIN_EXACT)
    return rep


@pytest.mark.parametrize("dtype", [sc.BF16, sc.F16])
def test_multiply_after_cast_bar_rejects_the_other_branch(dtype):
    from tests import parity
    case = _flag_case(dtype)
    res_false = oracle.run_case(case)
    case.multiply_before_cast = True
    res_true = oracle.run_case(case)
    case.multiply_before_cast = False
    assert res_false.status == 0 and res_true.status == 0
    rep = _check_q(case, res_false.q_out[0], res_false, parity)
    assert rep["q_exact_rate"] == 1.0
    assert rep["q_wide_rate"] < 0.05
    with pytest.raises(AssertionError):
        _check_q(case, res_true.q_out[0], res_false, parity)


@pytest.mark.parametrize("dtype", [sc.BF16, sc.F16])
def test_near_midpoint_marks_values_next_to_a_midpoint(dtype):
    from tests import parity
    q = brute.ulp_f16 if dtype == sc.F16 else brute.ulp_bf16
    base = np.array([1.0, 1.5, 3.0, 0.75, 2.0 ** -10])
    mid = base + 0.5 * q(base)
    assert parity.near_midpoint(mid, dtype).all()
    assert parity.near_midpoint(mid * (1 + 2.0 ** -20), dtype).all()
    assert not parity.near_midpoint(mid * (1 + 2.0 ** -16), dtype).any()
    assert not parity.near_midpoint(base, dtype).any()
    assert not parity.near_midpoint(np.array([0.0, np.nan]), dtype).any()

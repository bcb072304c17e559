"""Element-by-element comparison of the HIP path with the CPU oracle.

The bar:
* bit-exact: every cache element outside the rows written, every V element,
  the un-roped dims of the rope-only op, every radd result, q_output guard
  rows and padding columns, and the input buffer (unchanged);
* computed values (rotated and/or normalised):
    fp32:  |gpu - v| <= 1e-5 * max(|v|, m)
    bf16:  |gpu - v| <= ulps * ulp_bf16(max(|v|, 2^-8 * m))
    f16:   |gpu - v| <= ulps * ulp_f16(max(|v|, 2^-11 * m))
    FP8 cache rows (codes c, scale s): |c * s - v| <= s * ulp_e4m3(|v| / s)
           (+ 2^-8 of the row's largest |v| with bf16 scales, whose rounding
           can clamp the top code), and s within 2^-20 (f32) or one bf16 ulp
           of the oracle's scale; V rows and radd rows bit for bit (the same
           binary32 decisions on the same values)
  with v the oracle's unrounded value and m the length of v's RoPE pair
  (|v| for unrotated elements).  The pair-length floor is there because
  x*cos - y*sin can cancel: a bound relative to |v| alone would demand more
  than binary32 arithmetic can give.  ulps = 1 ("one ulp of the 16-bit
  type on a value computed in binary32").
* normalised rows with multiply_before_cast = false: the same one-ulp bar,
  except where the first intermediate rounding is ambiguous.  Each value
  passes two roundings to the 16-bit type before the rotation (n = dtype(x r),
  then m = dtype(n g) with g = dtype(gamma + w)).  Given n, both sides get
  the same m: g is exact on both (a sum of two 16-bit values rounds once),
  and n g is exact in binary32 (at most 22 significant bits).  n itself
  comes from the kernel's binary32 x r, whose relative error stays below
  2^-19.9: a sum of squares of at most 32 roundings per row (2^-19),
  halved by the root, one rounding of eps, v_rsq's ulp and the product.  So
  n can differ only where the exact x r lies within that distance of a
  rounding midpoint.  The oracle records x r (trace q_pre / k_pre); an
  element whose x r, or whose RoPE partner's, lies within 2^-18 (relative)
  of a midpoint of the type is checked against the wider bar below, every
  other one against one ulp, and at least 99 % of the latter must equal
  the oracle's rounding (when there are 1000 or more).  A kernel that ignored the flag (one
  rounding) fails both: only about 63 % of its values equal the
  twice-rounded ones.  The wider bar: 5 ulps of the 16-bit type at the
  scale of max(|v|, m).  A flipped n moves by one ulp; times g that moves
  m's input by up to 2 ulps of its result, and the second rounding can
  differ by one more: 3 ulps of a value no larger than m.  The rotation
  carries both values' errors (|c| + |s| <= sqrt 2) and the final rounding
  adds half an ulp: 4.75 ulps at the scale of m, however small cancellation
  makes |v|.  FP8 rows holding such an element keep their scale within 10
  ulps of the input type, relative (the row's largest value moves by up to
  5 ulps at sqrt 2 times its size), and their codes are checked at the
  GPU's own scale as above, plus those 5 ulps at the scale of m (5 eps m);
  the other FP8 rows get the plain FP8 bar.
"""
from __future__ import annotations

import numpy as np
import torch

from synth import cases as sc
from tests import brute
from tests import gpu_harness as gh


class Report(dict):
    pass


def tol_ok(gpu_bits: np.ndarray, exact: np.ndarray, mag: np.ndarray, dtype: str, ulps: int,
           floor: float = None):
    """``floor``: the fraction of the pair length m below which |v| is not
    taken as the scale (default 2^-11 for f16, 2^-8 for bf16)."""
    g = sc.bits_to_f64(gpu_bits, dtype)
    if dtype == sc.F32:
        tol = 1e-5 * np.maximum(np.abs(exact), mag)
    elif dtype == sc.F16:
        f = 2.0 ** -11 if floor is None else floor
        tol = ulps * brute.ulp_f16(np.maximum(np.abs(exact), f * mag))
    else:
        f = 2.0 ** -8 if floor is None else floor
        tol = ulps * brute.ulp_bf16(np.maximum(np.abs(exact), f * mag))
    return np.abs(g - exact) <= tol


# Relative distance from a rounding midpoint within which the kernel's
# binary32 x r (relative error below 2^-19.9) may round the other way.
MIDPOINT_BAND = 2.0 ** -18
# Wider bar for elements next to such a midpoint (multiply_before_cast off).
FLIP_ULPS = 5
# Smallest share of normalised multiply_before_cast-off values that must
# equal the oracle's rounding.
MBC_OFF_MIN_EXACT = 0.99
MIN_RATE_SAMPLE = 1000


def near_midpoint(pre: np.ndarray, dtype: str) -> np.ndarray:
    """Elements whose unrounded value lies within MIDPOINT_BAND (relative)
    of a rounding midpoint of the 16-bit ``dtype`` (never for binary32,
    whose bar is relative)."""
    pre = np.asarray(pre, dtype=np.float64)
    if dtype == sc.F32:
        return np.zeros(pre.shape, dtype=bool)
    q = brute.ulp_f16(pre) if dtype == sc.F16 else brute.ulp_bf16(pre)
    a = np.abs(pre)
    frac = a / q - np.floor(a / q)
    dist = np.abs(frac - 0.5) * q
    return np.isfinite(pre) & (a > 0) & (dist <= MIDPOINT_BAND * a)


def flip_mask(pre: np.ndarray, dtype: str, D: int, R: int, interleaved: bool,
              tail: bool) -> np.ndarray:
    """Rows [N, D] of x r -> the outputs that may take a flipped first
    rounding: the element's own, or its RoPE partner's."""
    near = near_midpoint(pre, dtype)
    out = near.copy()
    r0 = D - R if tail else 0
    j = np.arange(r0, r0 + R)
    if interleaved:
        partner = j ^ 1
    else:
        partner = np.where(j - r0 < R // 2, j + R // 2, j - R // 2)
    out[:, j] |= near[:, partner]
    return out


def check_rows(gpu: np.ndarray, ora: np.ndarray, exact: np.ndarray, mag: np.ndarray,
               copy_cols: np.ndarray, dtype: str, ulps: int, what: str, rep: Report,
               floor: float = None, wide: np.ndarray = None, min_exact: float = None):
    """Rows [N, D]: copy columns bit-exact, the others within tolerance.
    ``wide`` [N, D]: elements held to FLIP_ULPS at the scale of max(|v|, m)
    instead; ``min_exact``: the least share of computed values that must
    equal the oracle's rounding."""
    if gpu.size == 0:
        return
    assert np.array_equal(gpu[:, copy_cols], ora[:, copy_cols]), f"{what}: copied dims differ"
    comp = ~copy_cols
    g, o = gpu[:, comp], ora[:, comp]
    ok = tol_ok(g, exact[:, comp], mag[:, comp], dtype, ulps, floor)
    if wide is not None:
        w = wide[:, comp]
        ok_wide = tol_ok(g, exact[:, comp], mag[:, comp], dtype, FLIP_ULPS, 1.0)
        ok = np.where(w, ok_wide, ok)
        rep[what + "_wide_rate"] = float(w.mean()) if w.size else 0.0
    if not ok.all():
        bad = np.argwhere(~ok)[:5]
        det = [(int(r), int(c), float(sc.bits_to_f64(g[r, c], dtype)), float(exact[:, comp][r, c]),
                float(mag[:, comp][r, c])) for r, c in bad]
        raise AssertionError(f"{what}: {int((~ok).sum())} values out of tolerance, e.g. {det}")
    rate = float((g == o).mean()) if g.size else 1.0
    if min_exact is not None:
        # over the elements held to one ulp, once there are enough of them
        # for a rate to mean something
        narrow = ~wide[:, comp] if wide is not None else np.ones(g.shape, dtype=bool)
        if narrow.sum() >= MIN_RATE_SAMPLE:
            nrate = float((g[narrow] == o[narrow]).mean())
            assert nrate >= min_exact, (f"{what}: only {nrate:.4f} of the values equal the "
                                        f"oracle's rounding (at least {min_exact} required)")
    rep[what + "_exact_rate"] = rate
    rep[what + "_n"] = int(g.size)


def check_fp8_rows(codes: np.ndarray, scales: np.ndarray, ora_codes: np.ndarray,
                   ora_scales: np.ndarray, exact: np.ndarray, scale_dtype: str, what: str,
                   rep: Report, flip_eps=0.0, mag: np.ndarray = None):
    """FP8 rows [N, D] with their scale bits [N]: each dequantized value within
    one E4M3 step (at the GPU's own scale) of the oracle's unrounded value,
    each scale close to the oracle's.  ``flip_eps``: a scalar, or one value
    per row (0 for rows without a possibly flipped intermediate rounding)."""
    if codes.size == 0:
        return
    s = sc.bits_to_f64(scales, scale_dtype)[:, None]
    so = sc.bits_to_f64(ora_scales, scale_dtype)[:, None]
    deq = brute.e4m3_to_f64(codes) * s
    safe = np.where(s > 0, s, 1.0)
    tol = s * brute.ulp_e4m3(np.abs(exact) / safe)
    if scale_dtype == sc.BF16:
        tol = tol + 2.0 ** -8 * np.max(np.abs(exact), axis=1, keepdims=True)
    fe = np.broadcast_to(np.asarray(flip_eps, dtype=np.float64), (codes.shape[0],))[:, None]
    if np.any(fe):
        # the value before quantization: 5 ulps of the input type at the
        # pair's scale (5 eps m bounds them)
        tol = tol + FLIP_ULPS * fe * mag
    ok = np.abs(deq - exact) <= tol
    if not ok.all():
        bad = np.argwhere(~ok)[:5]
        det = [(int(r), int(c), float(deq[r, c]), float(exact[r, c]), float(s[r, 0]))
               for r, c in bad]
        raise AssertionError(f"{what}: {int((~ok).sum())} FP8 values out of tolerance, e.g. {det}")
    srel = (2.0 ** -20 if scale_dtype == sc.F32 else 2.0 ** -7) + 2 * FLIP_ULPS * fe
    sok = np.abs(s - so) <= srel * np.maximum(so, 1e-30)
    assert sok.all(), f"{what}: scales differ from the oracle's: {s[~sok][:5]} vs {so[~sok][:5]}"
    rep[what + "_code_exact_rate"] = float((codes == ora_codes).mean())
    rep[what + "_n"] = int(codes.size)


def _copy_cols(D: int, R: int, normed: bool, tail: bool = False) -> np.ndarray:
    """Dims that move unchanged: those outside the rotated range (the first
    R dims, or the last R with rope_tail), none after a norm."""
    cols = np.zeros(D, dtype=bool)
    if not normed:
        if tail:
            cols[:D - R] = True
        else:
            cols[R:] = True
    return cols


def bands_of(case):
    """(q_out index, cache index, n_q_heads, q normed, k normed, has V) per band."""
    if case.op == "store":
        return [(0, 0, case.n_q_heads, False, False, True)]
    if case.op == "bshd":
        return [(0, 0, case.n_q_heads, False, False, False)]
    if case.op in ("norm", "dual"):
        return [(i, b.cache, b.n_q_heads, b.q_gamma is not None, b.k_gamma is not None,
                 b.v_col >= 0) for i, b in enumerate(case.bands)]
    return []


def compare(case, dc: gh.DeviceCase, res, ulps: int = 1, untouched_pages: bool = True) -> Report:
    """Full comparison of one GPU call (already run) against the oracle result.
    ``untouched_pages=False`` skips the whole-pool sentinel count on compacted
    pools (for a pool other writers share)."""
    assert res.status == 0, f"oracle status {res.status}"
    rep = Report()
    # normalised rows rounded before the rotation (multiply_before_cast off):
    # elements next to a midpoint of the first rounding get the wider bar
    mbc_off = case.op in ("norm", "dual") and not case.multiply_before_cast
    eps_in = {sc.F32: 2.0 ** -23, sc.BF16: 2.0 ** -7, sc.F16: 2.0 ** -10}[case.dtype]

    def wide_of(pre, D):
        return flip_mask(pre.reshape(-1, D), case.dtype, D, case.rope_dim, case.interleaved,
                         case.rope_tail)
    dt = case.dtype
    qdt = case.q_dtype
    T = case.T
    # the input buffer is unchanged
    if case.buf.size:
        assert np.array_equal(gh.to_numpy_bits(dc.buf, dt), case.buf), "input buffer modified"
    # ---- Q outputs ----
    for qi, ci, Hq, qn, kn, hv in bands_of(case):
        D = case.caches[ci].head_dim
        full = gh.to_numpy_bits(dc.q_out[qi], qdt)
        g = gh.GUARD
        qsent = sc.SENTINEL[qdt]
        assert np.all(full[:g] == qsent) and np.all(full[g + T:] == qsent), \
            "q_output guard rows written"
        rows = full[g:g + T]
        ora = res.q_out[qi]
        stride = ora.shape[1]
        assert np.array_equal(rows[:, Hq * D:stride], ora[:, Hq * D:]), "q_output padding written"
        if case.op == "bshd" and T:
            # rows at or past a sequence's valid length: the input row, bit for bit
            S = case.seq_len
            pad = (np.arange(T) % S) >= np.repeat(np.asarray(case.lengths, np.int64), S)
            assert np.array_equal(rows[pad], case.buf[pad]), "a padded row is not the input row"
            rep["q_passed_rows"] = int(pad.sum())
        if Hq and T:
            tr = res.traces[qi]
            off_q = qn and mbc_off
            check_rows(rows[:, :Hq * D].reshape(-1, D), ora[:, :Hq * D].reshape(-1, D),
                       tr["q_exact"].reshape(-1, D), tr["q_mag"].reshape(-1, D),
                       _copy_cols(D, case.rope_dim, qn, case.rope_tail), qdt, ulps, f"q{qi}", rep,
                       wide=wide_of(tr["q_pre"], D) if off_q else None,
                       min_exact=MBC_OFF_MIN_EXACT if off_q and qdt != sc.F32 else None)
    # ---- caches ----
    for ci, dcache in enumerate(dc.caches):
        host = dcache.host
        ora_pool = res.pools[ci]
        pages = res.page_maps[ci]
        if pages is None:
            pages = np.arange(host.num_pages)
        gpu_pool = dcache.pages(pages)
        D = host.head_dim
        fp8 = host.dtype == sc.FP8
        g_flat = gpu_pool.reshape(-1).copy()
        o_flat = ora_pool.reshape(-1).copy()
        if fp8:
            gs_flat = dcache.scale_pages(pages).reshape(-1).copy()
            os_flat = res.scales[ci].reshape(-1).copy()
        for qi, cj, Hq, qn, kn, hv in bands_of(case):
            if cj != ci or T == 0:
                continue
            tr = res.traces[qi]
            koff = tr["k_row_off"].reshape(-1)
            live = koff >= 0                       # rows the op wrote (bshd: real rows only)
            idx = koff[live][:, None] + np.arange(D)[None, :]
            off_k = kn and mbc_off
            wide = wide_of(tr["k_pre"], D)[live] if off_k else None
            if fp8:
                soff = tr["k_scale_off"].reshape(-1)[live]
                row_eps = wide.any(axis=1) * eps_in if off_k else 0.0
                check_fp8_rows(g_flat[idx], gs_flat[soff], o_flat[idx], os_flat[soff],
                               tr["k_exact"].reshape(-1, D)[live], host.scale_dtype, f"k{qi}",
                               rep, row_eps, tr["k_mag"].reshape(-1, D)[live])
                gs_flat[soff] = 0
                os_flat[soff] = 0
            else:
                check_rows(g_flat[idx], o_flat[idx], tr["k_exact"].reshape(-1, D)[live],
                           tr["k_mag"].reshape(-1, D)[live], _copy_cols(D, case.rope_dim, kn, case.rope_tail),
                           dt, ulps, f"k{qi}", rep, wide=wide,
                           min_exact=MBC_OFF_MIN_EXACT if off_k and dt != sc.F32 else None)
            # written K rows are checked: blank them before the bitwise comparison
            g_flat[idx] = 0
            o_flat[idx] = 0
        if fp8 and not np.array_equal(gs_flat, os_flat):
            bad = np.flatnonzero(gs_flat != os_flat)
            raise AssertionError(f"cache {ci}: {len(bad)} scales differ outside the checked K "
                                 f"rows, first at {bad[:5]} gpu={gs_flat[bad[:5]]} "
                                 f"oracle={os_flat[bad[:5]]}")
        if not np.array_equal(g_flat, o_flat):
            bad = np.flatnonzero(g_flat != o_flat)
            raise AssertionError(f"cache {ci}: {len(bad)} elements differ outside the checked K "
                                 f"rows, first at flat {bad[:5]} "
                                 f"gpu={g_flat[bad[:5]]} oracle={o_flat[bad[:5]]}")
        if res.page_maps[ci] is not None and untouched_pages:
            # pages the batch does not touch must hold nothing but the sentinel
            n_dev = int((dcache.pool != gh.sentinel_int(host.dtype)).sum().item())
            n_touched = int((gpu_pool != sc.SENTINEL[host.dtype]).sum())
            assert n_dev == n_touched, "a page outside the batch was written"
    return rep

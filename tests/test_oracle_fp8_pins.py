"""Pins of the oracle's FP8 (OCP E4M3) cache rows and of the Q output dtype.

The encoding is pinned to the format's definition: golden cases with their
reasons (tests/golden/e4m3_rne_cases.txt, OCP OFP8 specification, E4M3),
an exhaustive decode from the bit fields and a neighbour search for the
rounding.  The quantization of a row (one scale per written head row, every
decision in binary32 -- a reading: the pages name a cache collection's scale
dtype and quantization granularity without defining them) is pinned by an
independent numpy-binary32 implementation with neighbour-search codes: V
rows and radd results must match it bit for bit, roped K rows within one
E4M3 step of the exact value.  The Q output dtype of the store op
(rope_split_store_paged_ragged page, Parameters: q_out_dtype) is pinned by
brute force in every dtype pair.
"""
from __future__ import annotations

import os

import numpy as np
import pytest

import oracle
from synth import cases as sc
from tests import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# the encoding
# --------------------------------------------------------------------------

def test_e4m3_rounding_golden_cases():
    n = 0
    with open(os.path.join(GOLDEN, "e4m3_rne_cases.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            val, code = line.split()[:2]
            assert oracle.round_e4m3(float.fromhex(val)) == int(code, 16), line
            n += 1
    assert n >= 20


def test_e4m3_decode_matches_bit_fields():
    codes, vals = brute.e4m3_table()
    for c, v in zip(codes, vals):
        got = oracle.e4m3_to_double(int(c))
        assert got == v and np.signbit(got) == bool(c & 0x80), hex(c)
    assert np.isnan(oracle.e4m3_to_double(0x7F)) and np.isnan(oracle.e4m3_to_double(0xFF))
    # every finite code round-trips
    for c in codes:
        assert oracle.round_e4m3(oracle.e4m3_to_double(int(c))) == int(c), hex(c)


def test_e4m3_rounding_matches_neighbour_search():
    _, vals = brute.e4m3_table()
    fin = np.unique(vals[vals >= 0])
    rng = np.random.default_rng(17)
    xs = list(rng.standard_normal(2000) * 40) + list(rng.standard_normal(500) * 0.01)
    xs += list((fin[:-1] + fin[1:]) / 2)                        # every tie
    xs += list(-(fin[:-1] + fin[1:]) / 2)
    xs += list(rng.uniform(440, 470, 50))                       # around saturation
    for x in xs:
        assert oracle.round_e4m3(float(x)) == brute.nearest_even_e4m3(float(x)), float(x).hex()


# --------------------------------------------------------------------------
# quantized cache rows
# --------------------------------------------------------------------------

def _fp8_store(scale_dtype=sc.F32, interleaved=True, dtype=sc.BF16, R=64, seed=51, q_out=None,
               lengths=(3, 0, 6, 2), clen=(0, 7, 2, 30)):
    return sc.make_store_case("fp8pin", seed, dtype, list(lengths), list(clen), Hq=3, Hk=2, D=64,
                              rope_dim=R, interleaved=interleaved, theta=1e4, max_seq_len=64,
                              P=8, L=2, layer=1, cache_dtype=sc.FP8, scale_dtype=scale_dtype,
                              q_out_dtype=q_out)


def _rows(case):
    for t, b, cseq, pos in brute.walk_tokens(case):
        page, slot = brute.page_slot(case.caches[0], cseq, pos)
        yield t, pos, page, slot


def _scale_value(bits, scale_dtype):
    return float(sc.bits_to_f64(np.array([bits], dtype=sc.BITS_DTYPE[scale_dtype]), scale_dtype)[0])


@pytest.mark.parametrize("scale_dtype", [sc.F32, sc.BF16])
@pytest.mark.parametrize("dtype", [sc.F32, sc.BF16, sc.F16])
def test_fp8_store_v_rows_match_binary32_quantization_exactly(dtype, scale_dtype):
    case = _fp8_store(scale_dtype=scale_dtype, dtype=dtype)
    res = oracle.run_case(case)
    assert res.status == 0
    c = case.caches[0]
    D, Hq, Hk = c.head_dim, case.n_q_heads, c.num_kv_heads
    pool, scl = res.pools[0], res.scales[0]
    for t, pos, page, slot in _rows(case):
        for h in range(Hk):
            v = sc.bits_to_f64(case.buf[t, (Hq + Hk + h) * D:(Hq + Hk + h + 1) * D], dtype)
            codes, sbits = brute.quantize_row_f32(v, scale_dtype)
            assert np.array_equal(pool[page, 1, case.layer_idx, slot, h], codes), (t, h)
            assert scl[page, 1, case.layer_idx, slot, h] == sbits, (t, h)


@pytest.mark.parametrize("scale_dtype", [sc.F32, sc.BF16])
@pytest.mark.parametrize("interleaved", [True, False])
def test_fp8_store_k_rows_are_the_quantized_rotation(interleaved, scale_dtype):
    case = _fp8_store(scale_dtype=scale_dtype, interleaved=interleaved, R=32)
    res = oracle.run_case(case)
    assert res.status == 0
    c = case.caches[0]
    D, Hq, Hk, R = c.head_dim, case.n_q_heads, c.num_kv_heads, case.rope_dim
    pool, scl = res.pools[0], res.scales[0]
    written = np.zeros(pool.shape[:5], dtype=bool)
    for t, pos, page, slot in _rows(case):
        for h in range(Hk):
            x = sc.bits_to_f64(case.buf[t, (Hq + h) * D:(Hq + h + 1) * D], case.dtype)
            y, _ = brute.rope_complex(x, case.freqs[pos], R, case.interleaved)
            codes, sbits = brute.quantize_row_f32(y, scale_dtype)
            got_codes = pool[page, 0, case.layer_idx, slot, h]
            got_s = _scale_value(scl[page, 0, case.layer_idx, slot, h], scale_dtype)
            # the same decisions on the same binary32 values: the same bits
            assert np.array_equal(got_codes, codes), (t, h)
            assert scl[page, 0, case.layer_idx, slot, h] == sbits
            # and the dequantized row is within one E4M3 step of the rotation
            deq = brute.e4m3_to_f64(got_codes) * got_s
            assert np.all(np.abs(deq - y) <= got_s * brute.ulp_e4m3(y / got_s)), (t, h)
            written[page, :, case.layer_idx, slot, h] = True
    # rows the batch does not reach keep the sentinel, codes and scales alike
    assert np.all(pool[~written] == sc.SENTINEL[sc.FP8])
    assert np.all(scl[~written] == sc.SENTINEL[scale_dtype])


def test_fp8_zero_row_has_zero_scale_and_keeps_signs():
    case = _fp8_store(lengths=(2,), clen=(0,))
    Hq, Hk, D = 3, 2, 64
    case.buf[0, (Hq + Hk) * D:(Hq + Hk + 1) * D] = sc.to_bits(np.zeros(D), sc.BF16)
    case.buf[0, (Hq + Hk) * D + 5] = 0x8000                       # -0
    res = oracle.run_case(case)
    page, slot = brute.page_slot(case.caches[0], 0, 0)
    codes = res.pools[0][page, 1, 1, slot, 0]
    assert codes[5] == 0x80 and np.all(np.delete(codes, 5) == 0)
    assert res.scales[0][page, 1, 1, slot, 0] == 0


def test_fp8_radd_is_dequantize_add_requantize_bit_for_bit():
    case = sc.make_radd_case("fp8radd", 53, sc.BF16, [4, 0, 3], [5, 1, 9, 0, 12], 1, Hk=2, D=64,
                             P=8, L=2, layer=1, cache_dtype=sc.FP8, a_std=0.05)
    c = case.caches[0]
    before, s_before = c.materialize(), c.materialize_scales()
    res = oracle.run_case(case)
    assert res.status == 0
    D, Hk = c.head_dim, c.num_kv_heads
    for t, b, cseq, pos in brute.walk_tokens(case):
        page, slot = brute.page_slot(c, cseq, pos)
        for plane in (0, 1):
            for h in range(Hk):
                s = np.float32(_scale_value(s_before[page, plane, 1, slot, h], sc.F32))
                cur = brute.e4m3_to_f64(before[page, plane, 1, slot, h]).astype(np.float32) * s
                a = sc.bits_to_f64(case.buf[t, plane * Hk * D + h * D:plane * Hk * D + (h + 1) * D],
                                   sc.BF16).astype(np.float32)
                codes, sbits = brute.quantize_row_f32((cur + a).astype(np.float64), sc.F32)
                assert np.array_equal(res.pools[0][page, plane, 1, slot, h], codes), (t, plane, h)
                assert res.scales[0][page, plane, 1, slot, h] == sbits


def test_fp8_in_place_norm_rope_reads_the_dequantized_row():
    case = sc.make_norm_case("fp8norm", 54, sc.BF16, [3, 5], [2, 0], Hq=2, Hk=2, D=64, rope_dim=64,
                             interleaved=False, theta=1e4, max_seq_len=64, P=8, L=1, layer=0,
                             k_in_cache=True, cache_dtype=sc.FP8, scale_dtype=sc.BF16)
    c = case.caches[0]
    before, s_before = c.materialize(), c.materialize_scales()
    res = oracle.run_case(case)
    assert res.status == 0
    band = case.bands[0]
    g = sc.bits_to_f64(band.k_gamma, sc.BF16)
    for t, b, cseq, pos in brute.walk_tokens(case):
        page, slot = brute.page_slot(c, cseq, pos)
        for h in range(c.num_kv_heads):
            s = np.float32(_scale_value(s_before[page, 0, 0, slot, h], sc.BF16))
            x = (brute.e4m3_to_f64(before[page, 0, 0, slot, h]).astype(np.float32) * s)
            x = x.astype(np.float64)
            n = x / np.sqrt(np.mean(x * x) + band.epsilon) * g
            y, _ = brute.rope_complex(n, case.freqs[pos], case.rope_dim, case.interleaved)
            got_s = _scale_value(res.scales[0][page, 0, 0, slot, h], sc.BF16)
            deq = brute.e4m3_to_f64(res.pools[0][page, 0, 0, slot, h]) * got_s
            # one E4M3 step, plus the bf16 scale's rounding when it clamps the top code
            tol = got_s * brute.ulp_e4m3(y / got_s) + np.max(np.abs(y)) * 2.0 ** -8
            assert np.all(np.abs(deq - y) <= tol), (t, h)


# --------------------------------------------------------------------------
# Q output dtype
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,q_out", [(sc.F32, sc.BF16), (sc.F32, sc.F16), (sc.BF16, sc.F32),
                                         (sc.F16, sc.BF16), (sc.BF16, sc.F16)])
def test_q_output_dtype_rounds_roped_and_converts_the_rest(dtype, q_out):
    case = sc.make_store_case("qout", 55, dtype, [4, 3], [0, 9], Hq=3, Hk=1, D=64, rope_dim=32,
                              interleaved=True, theta=1e4, max_seq_len=64, P=8, L=1, layer=0,
                              q_out_dtype=q_out)
    res = oracle.run_case(case)
    assert res.status == 0
    D, R = 64, 32
    q = res.q_out[0]
    assert q.dtype == sc.BITS_DTYPE[q_out]
    for t, b, cseq, pos in brute.walk_tokens(case):
        for h in range(3):
            x = sc.bits_to_f64(case.buf[t, h * D:(h + 1) * D], dtype)
            y, mag = brute.rope_complex(x, case.freqs[pos], R, True)
            got = sc.bits_to_f64(q[t, h * D:(h + 1) * D], q_out)
            # roped: one rounding to q_out (half its ulp, relative to the pair length)
            ulp = {sc.F32: 2.0 ** -23, sc.BF16: 2.0 ** -7, sc.F16: 2.0 ** -10}[q_out]
            assert np.all(np.abs(got[:R] - y[:R]) <= ulp * mag[:R]), (t, h)
            # the rest: the input value converted to q_out by nearest-even
            assert np.array_equal(q[t, h * D + R:(h + 1) * D], sc.to_bits(x[R:], q_out)), (t, h)

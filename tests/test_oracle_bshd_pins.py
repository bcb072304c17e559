"""Pins of the oracle's padded continuous-batching op against things other
than itself (generic_fused_qk_rope_bshd_continuous_batch page, signature and
Args).

* brute force: every row of every sequence is walked by (b, s) -- not by
  the oracle's loops -- real rows rotated by Python complex multiplication
  at position cache_lengths[b] + s, the K row found by numpy indexing of the
  pool's logical shape and compared with the pool before the call;
* rows at or past a sequence's valid length come out as the input's bits
  and leave the cache alone (the reading taken of "RoPE only within the
  valid lengths"), also when valid_lengths exceeds the padded length;
* position 0 is the identity (cos 0 = 1, sin 0 = 0 in the table);
* every pool element other than the real rows' K rows keeps its bits;
* a real row whose position is out of range is an error, a padded one never.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from synth import cases as sc
from tests import brute


def _case(dtype=sc.BF16, interleaved=True, valid=(3, 0, 7, 9), S=6, clen=(0, 4, 11, 2),
          D=64, R=64, Hq=3, Hk=2, capacity=32, L=2, layer=1, seed=31, freq_dtype=None,
          max_seq_len=40, num_blocks=None):
    return sc.make_bshd_case("bshd_pin", seed, dtype, list(valid), S, list(clen), Hq=Hq, Hk=Hk,
                             D=D, rope_dim=R, interleaved=interleaved, theta=1e4,
                             max_seq_len=max_seq_len, capacity=capacity, L=L, layer=layer,
                             num_blocks=num_blocks, freq_dtype=freq_dtype)


def _check_against_brute(case, res, pair_tol):
    cache = case.caches[0]
    D, Hk, Hq, R, S = cache.head_dim, cache.num_kv_heads, case.n_q_heads, case.rope_dim, case.seq_len
    before = cache.materialize()
    pool, out = res.pools[0], res.q_out[0]
    written = np.zeros(before.shape[:5], dtype=bool)
    for b, vl in enumerate(case.lengths):
        for s in range(S):
            t = b * S + s
            if s >= vl:
                assert np.array_equal(out[t], case.buf[t]), (b, s)
                continue
            pos = int(cache.cache_lengths[b]) + s
            page, slot = brute.page_slot(cache, b, pos)
            frow = case.freqs[pos]
            for h in range(Hq):
                x_bits = case.buf[t, h * D:(h + 1) * D]
                y, mag = brute.rope_complex(brute.as_f64(x_bits, case.dtype), frow, R,
                                            case.interleaved)
                got_bits = out[t, h * D:(h + 1) * D]
                got = brute.as_f64(got_bits, case.dtype)
                assert np.all(np.abs(got[:R] - y[:R]) <= pair_tol * mag[:R]), (b, s, h)
                assert np.array_equal(got_bits[R:], x_bits[R:]), (b, s, h)
            for h in range(Hk):
                x_bits = before[page, 0, case.layer_idx, slot, h]
                y, mag = brute.rope_complex(brute.as_f64(x_bits, case.dtype), frow, R,
                                            case.interleaved)
                got_bits = pool[page, 0, case.layer_idx, slot, h]
                got = brute.as_f64(got_bits, case.dtype)
                assert np.all(np.abs(got[:R] - y[:R]) <= pair_tol * mag[:R]), (b, s, h)
                assert np.array_equal(got_bits[R:], x_bits[R:]), (b, s, h)
                written[page, 0, case.layer_idx, slot, h] = True
    # every other pool element (V rows, padded positions, other layers) kept its bits
    assert np.array_equal(pool[~written], before[~written])
    return int(written.sum())


TOL = {sc.F32: 2.0 ** -23, sc.BF16: 2.0 ** -8, sc.F16: 2.0 ** -11}


@pytest.mark.parametrize("interleaved", [True, False])
@pytest.mark.parametrize("dtype", [sc.F32, sc.BF16, sc.F16])
def test_bshd_matches_complex_brute_force(dtype, interleaved):
    case = _case(dtype=dtype, interleaved=interleaved)
    res = oracle.run_case(case)
    assert res.status == 0
    n = _check_against_brute(case, res, TOL[dtype])
    real = sum(min(int(v), case.seq_len) for v in case.lengths)
    assert n == real * case.caches[0].num_kv_heads


@pytest.mark.parametrize("interleaved", [True, False])
def test_bshd_partial_rope_other_table_types_and_long_valid_lengths(interleaved):
    # valid length 9 > padded length 6: every row of that sequence is real
    for fdt in (sc.F32, sc.F16):
        case = _case(dtype=sc.BF16, interleaved=interleaved, R=32, freq_dtype=fdt)
        res = oracle.run_case(case)
        assert res.status == 0
        _check_against_brute(case, res, TOL[sc.BF16])


def test_bshd_padded_rows_are_copied_bit_for_bit():
    case = _case(dtype=sc.F32, valid=(0, 2, 0, 6), clen=(30, 0, 5, 1))
    # special values in the padded rows of sequences 0 and 2 survive untouched
    sv = np.array([0x7FC00001, 0x7F800001, 0xFF800000, 0x80000000, 0x00000001], np.uint32)
    S = case.seq_len
    for b in (0, 2):
        flat = case.buf[b * S:(b + 1) * S].reshape(-1)      # a view of the padded rows
        flat[::7] = sv[np.arange(flat[::7].size) % len(sv)]
    res = oracle.run_case(case)
    assert res.status == 0
    for b in (0, 2):
        assert np.array_equal(res.q_out[0][b * S:(b + 1) * S], case.buf[b * S:(b + 1) * S])
    _check_against_brute(case, res, TOL[sc.F32])


def test_bshd_position_zero_is_identity():
    case = _case(dtype=sc.BF16, valid=(1, 1, 1), S=2, clen=(0, 0, 0))
    res = oracle.run_case(case)
    assert res.status == 0
    cache, S = case.caches[0], case.seq_len
    before = cache.materialize()
    for b in range(3):
        assert np.array_equal(res.q_out[0][b * S], case.buf[b * S])
        page, slot = brute.page_slot(cache, b, 0)
        assert np.array_equal(res.pools[0][page, 0, case.layer_idx, slot],
                              before[page, 0, case.layer_idx, slot])


def test_bshd_position_out_of_range_only_matters_for_real_rows():
    # sequence 1's real rows reach positions 38..41 >= max_seq_len 40
    bad = _case(valid=(3, 4), S=5, clen=(0, 38), max_seq_len=40, capacity=64)
    assert oracle.run_case(bad).status == -6
    # the same cache length with no real rows past the table is fine
    ok = _case(valid=(3, 2), S=5, clen=(0, 38), max_seq_len=40, capacity=64)
    assert oracle.run_case(ok).status == 0


def test_bshd_empty_grid_writes_nothing():
    case = _case(valid=(0, 0), S=4, clen=(1, 2))
    res = oracle.run_case(case)
    assert res.status == 0
    assert np.array_equal(res.q_out[0], case.buf)
    assert np.array_equal(res.pools[0], case.caches[0].materialize())

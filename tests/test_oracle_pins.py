"""Pins of the CPU oracle against facts that do not come from the oracle.

Each test ties one part of the oracle to the documentation pages, to
mathematics or to a brute-force computation written differently:

* bf16 rounding: hand-derived IEEE-754 cases (tests/golden) and exhaustive
  neighbour search; binary16 rounding: hand-derived cases and numpy's own
  float64 -> float16 conversion;
* RoPE: Python complex multiplication on the tiny fp32 workload, both
  layouts, partial rope; position 0 is the identity; every pair keeps its
  length; unit vectors give (cos, sin) of p * theta_i computed here with
  ``math``; the dot product of a roped query and key depends only on the
  position difference (the property RoPE is built for);
* half-split equals interleaved after permuting each head's halves;
* paged placement: rows land where walking the batch and indexing the pool
  by its logical shape says; an identity page table reproduces a dense
  [batch, seq, head, dim] cache; a permuted table moves rows, not values;
* copies: V rows and un-roped dims keep every bit, specials included; every
  pool element outside the written rows keeps its sentinel;
* RMSNorm: closed form for constant vectors, scale invariance, unit mean
  square, gamma/weight_offset interchange;
* radd: numpy binary32 adds, +0 / -0 leave the cache unchanged.
"""
from __future__ import annotations

import math
import os

import numpy as np
import pytest

import oracle
from synth import cases as sc
from tests import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# bf16 rounding
# --------------------------------------------------------------------------

def test_bf16_rounding_golden_cases():
    n = 0
    with open(os.path.join(GOLDEN, "bf16_rne_cases.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            val, bits = line.split()[:2]
            assert oracle.round_bf16(float.fromhex(val)) == int(bits, 16), line
            n += 1
    assert n >= 15


def test_bf16_rounding_matches_exhaustive_search():
    vals, bits = brute.bf16_table()
    rng = np.random.default_rng(123)
    xs = list(rng.standard_normal(3000))
    xs += list(rng.standard_normal(1000) * 1e-39)              # subnormal range
    xs += list(rng.standard_normal(500) * 1e38)                # near overflow
    # exact midpoints between neighbours (ties)
    idx = rng.integers(0, len(vals) - 1, 1000)
    xs += list((vals[idx] + vals[idx + 1]) / 2)
    for x in xs:
        x = float(x)
        assert oracle.round_bf16(x) == brute.nearest_even_bf16(x, vals, bits), x.hex()


def test_bf16_special_values():
    assert oracle.round_bf16(float("inf")) == 0x7F80
    assert oracle.round_bf16(float("-inf")) == 0xFF80
    nan = oracle.round_bf16(float("nan"))
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F) != 0 and (nan & 0x40)
    for b in (0x0000, 0x8000, 0x0001, 0x3F80, 0xC049, 0x7F7F):
        assert oracle.round_bf16(oracle.bf16_to_double(b)) == b


def test_f16_rounding_golden_cases():
    n = 0
    with open(os.path.join(GOLDEN, "f16_rne_cases.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            val, bits = line.split()[:2]
            assert oracle.round_f16(float.fromhex(val)) == int(bits, 16), line
            n += 1
    assert n >= 15


def test_f16_rounding_matches_numpy():
    # numpy's float64 -> float16 conversion is a separate, correctly rounded
    # (ties-to-even) implementation of the same IEEE operation
    rng = np.random.default_rng(7)
    xs = np.concatenate([rng.standard_normal(4000), rng.standard_normal(1000) * 1e-5,
                         rng.standard_normal(1000) * 3e4, rng.standard_normal(500) * 1e-7])
    every = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).view(np.float16)
    fin = np.sort(every[np.isfinite(every)].astype(np.float64))
    mids = (fin[:-1] + fin[1:]) / 2
    xs = np.concatenate([xs, rng.choice(mids, 2000)])
    for x in xs:
        want = int(np.float64(x).astype(np.float16).view(np.uint16))
        assert oracle.round_f16(float(x)) == want, float(x).hex()
    for h in (0x0000, 0x8000, 0x0001, 0x3C00, 0x4248, 0x7BFF, 0x0400):
        assert oracle.round_f16(oracle.f16_to_double(h)) == h


# --------------------------------------------------------------------------
# RoPE and paged placement against brute force
# --------------------------------------------------------------------------

def _store_case(interleaved=True, dtype=sc.F32, rope_dim=64, D=64, lengths=(3, 5),
                cache_lengths=(0, 4), P=16, num_pages=8, max_pages=4, seed=1, L=1, layer=0,
                specials=False, q_out_pad=0, row_pad=0, Hq=4, Hk=2, max_seq_len=64, theta=1e4):
    return sc.make_store_case("pin", seed, dtype, list(lengths), list(cache_lengths), Hq=Hq, Hk=Hk,
                              D=D, rope_dim=rope_dim, interleaved=interleaved, theta=theta,
                              max_seq_len=max_seq_len, P=P, L=L, layer=layer,
                              num_pages=num_pages, max_pages=max_pages, specials=specials,
                              q_out_pad=q_out_pad, row_pad=row_pad)


def _check_store_against_brute(case, res, pair_tol):
    """Every Q/K/V row of the oracle vs the complex-multiply brute force;
    returns the set of pool rows written, for the sentinel check."""
    cache = case.caches[0]
    D, Hk, Hq, R = cache.head_dim, cache.num_kv_heads, case.n_q_heads, case.rope_dim
    pool = res.pools[0]
    q_out = res.q_out[0]
    written = set()
    for t, b, cseq, pos in brute.walk_tokens(case):
        page, slot = brute.page_slot(cache, cseq, pos)
        frow = case.freqs[pos]
        row = case.buf[t]
        for h in range(Hq + Hk):
            x_bits = row[h * D:(h + 1) * D]
            y, mag = brute.rope_complex(brute.as_f64(x_bits, case.dtype), frow, R,
                                        case.interleaved)
            if h < Hq:
                got_bits = q_out[t, h * D:(h + 1) * D]
            else:
                got_bits = pool[page, 0, case.layer_idx, slot, h - Hq]
                written.add((page, 0, case.layer_idx, slot, h - Hq))
            got = brute.as_f64(got_bits, case.dtype)
            assert np.all(np.abs(got[:R] - y[:R]) <= pair_tol * mag[:R]), (t, h)
            # dims beyond rope_dim: the same bits
            assert np.array_equal(got_bits[R:], x_bits[R:]), (t, h)
        for h in range(Hk):
            v_bits = row[(Hq + Hk + h) * D:(Hq + Hk + h + 1) * D]
            assert np.array_equal(pool[page, 1, case.layer_idx, slot, h], v_bits), (t, h)
            written.add((page, 1, case.layer_idx, slot, h))
    return written


def _check_sentinels(case, pool, written):
    sent = sc.SENTINEL[case.dtype]
    mask = np.ones(pool.shape[:5], dtype=bool)
    for w in written:
        mask[w] = False
    assert np.all(pool[mask] == sent)


@pytest.mark.parametrize("interleaved", [True, False])
def test_tiny_store_matches_complex_brute_force(interleaved):
    case = sc.tiny_fp32() if interleaved else _store_case(interleaved=False)
    res = oracle.run_case(case)
    assert res.status == 0
    written = _check_store_against_brute(case, res, pair_tol=2.0 ** -23)
    assert len(written) == case.T * 2 * case.caches[0].num_kv_heads
    _check_sentinels(case, res.pools[0], written)


@pytest.mark.parametrize("interleaved", [True, False])
@pytest.mark.parametrize("dtype", [sc.F32, sc.BF16, sc.F16])
def test_partial_rope_and_ragged_batch_brute_force(interleaved, dtype):
    # empty sequences between non-empty ones, partial rope, multi-page rows,
    # several layers, padded row strides
    case = _store_case(interleaved=interleaved, dtype=dtype, rope_dim=32, D=64,
                       lengths=(0, 7, 0, 0, 19, 1, 0), cache_lengths=(3, 5, 0, 9, 14, 31, 2),
                       P=4, num_pages=40, max_pages=16, L=3, layer=1, q_out_pad=8, row_pad=16,
                       seed=11)
    res = oracle.run_case(case)
    assert res.status == 0
    tol = {sc.F32: 2.0 ** -23, sc.BF16: 2.0 ** -8, sc.F16: 2.0 ** -11}[dtype]
    written = _check_store_against_brute(case, res, pair_tol=tol)
    _check_sentinels(case, res.pools[0], written)
    # q_out padding columns untouched
    Hq, D = case.n_q_heads, case.caches[0].head_dim
    assert np.all(res.q_out[0][:, Hq * D:] == sc.SENTINEL[dtype])


@pytest.mark.parametrize("interleaved", [True, False])
@pytest.mark.parametrize("dtype", [sc.F32, sc.BF16])
def test_trailing_partial_rope_brute_force(interleaved, dtype):
    """rope_tail: the LAST rope_dim dims of each head rotate, the first
    D - rope_dim move as bits (the other convention for a partial rope)."""
    R, D = 32, 64
    case = sc.make_store_case("tail", 57, dtype, [5, 0, 9], [3, 2, 20], Hq=4, Hk=2, D=D,
                              rope_dim=R, interleaved=interleaved, theta=1e4, max_seq_len=64,
                              P=8, L=2, layer=1, rope_tail=True)
    res = oracle.run_case(case)
    assert res.status == 0
    tol = {sc.F32: 2.0 ** -23, sc.BF16: 2.0 ** -8}[dtype]
    cache = case.caches[0]
    Hq, Hk = 4, 2
    for t, b, cseq, pos in brute.walk_tokens(case):
        page, slot = brute.page_slot(cache, cseq, pos)
        for h in range(Hq + Hk):
            x_bits = case.buf[t, h * D:(h + 1) * D]
            y, mag = brute.rope_complex(brute.as_f64(x_bits[D - R:], dtype), case.freqs[pos], R,
                                        interleaved)
            got_bits = (res.q_out[0][t, h * D:(h + 1) * D] if h < Hq
                        else res.pools[0][page, 0, 1, slot, h - Hq])
            got = brute.as_f64(got_bits[D - R:], dtype)
            assert np.all(np.abs(got - y) <= tol * mag), (t, h)
            assert np.array_equal(got_bits[:D - R], x_bits[:D - R]), (t, h)


def test_trailing_rope_is_leading_rope_of_rolled_heads():
    """Rolling every head by D - R dims maps the trailing convention onto the
    leading one: the two runs agree bit for bit after rolling back."""
    R, D, Hq, Hk = 32, 64, 4, 2
    mk = lambda tail: sc.make_store_case("roll", 58, sc.BF16, [6, 4], [0, 11], Hq=Hq, Hk=Hk, D=D,
                                         rope_dim=R, interleaved=False, theta=1e4,
                                         max_seq_len=64, P=8, L=1, layer=0, rope_tail=tail)
    tail, lead = mk(True), mk(False)
    H = Hq + 2 * Hk
    lead.buf = np.ascontiguousarray(
        np.roll(tail.buf.reshape(tail.T, H, D), -(D - R), axis=2).reshape(tail.T, H * D))
    rt, rl = oracle.run_case(tail), oracle.run_case(lead)
    qt = rt.q_out[0].reshape(tail.T, Hq, D)
    ql = np.roll(rl.q_out[0].reshape(lead.T, Hq, D), D - R, axis=2)
    assert np.array_equal(qt, ql)
    kt = rt.pools[0][:, 0]
    kl = np.roll(rl.pools[0][:, 0], D - R, axis=-1)
    assert np.array_equal(kt, kl)


def test_position_zero_is_identity():
    case = _store_case(lengths=(1, 1, 1), cache_lengths=(0, 0, 0), num_pages=12, seed=5)
    res = oracle.run_case(case)
    Hq, Hk, D = 4, 2, 64
    assert np.array_equal(res.q_out[0], case.buf[:, :Hq * D])
    for t, b, cseq, pos in brute.walk_tokens(case):
        page, slot = brute.page_slot(case.caches[0], cseq, pos)
        k = case.buf[t, Hq * D:(Hq + Hk) * D].reshape(Hk, D)
        assert np.array_equal(res.pools[0][page, 0, 0, slot], k)


@pytest.mark.parametrize("dtype,tol", [(sc.F32, 1e-6), (sc.BF16, 2.0 ** -8)])
def test_rotation_keeps_pair_length(dtype, tol):
    case = _store_case(dtype=dtype, lengths=(20, 13), cache_lengths=(7, 30), max_seq_len=64,
                       num_pages=8, seed=9, max_pages=4)
    res = oracle.run_case(case)
    D, Hq = 64, 4
    x = brute.as_f64(case.buf[:, :Hq * D], dtype).reshape(-1, Hq, 32, 2)
    y = brute.as_f64(res.q_out[0], dtype).reshape(-1, Hq, 32, 2)
    nx = np.hypot(x[..., 0], x[..., 1])
    ny = np.hypot(y[..., 0], y[..., 1])
    assert np.all(np.abs(ny - nx) <= tol * nx + 1e-30)


@pytest.mark.parametrize("interleaved", [True, False])
def test_unit_vectors_give_cos_sin_closed_form(interleaved):
    R = D = 64
    base = 1e4
    lengths = [1] * 6
    positions = [0, 1, 2, 17, 40, 63]
    case = _store_case(interleaved=interleaved, lengths=lengths, cache_lengths=positions,
                       num_pages=24, max_pages=4, seed=3, Hq=R // 2, Hk=1)
    # Q head h = e_{j0(h)}: the real slot of frequency h
    buf = np.zeros_like(case.buf)
    one = sc.to_bits(np.array([1.0]), sc.F32)[0]
    for h in range(R // 2):
        j0 = 2 * h if interleaved else h
        buf[:, h * D + j0] = one
    case.buf = buf
    res = oracle.run_case(case)
    out = brute.as_f64(res.q_out[0], sc.F32).reshape(len(lengths), R // 2, D)
    for t, p in enumerate(positions):
        for i in range(R // 2):
            ang = p * base ** (-2.0 * i / R)
            j0, j1 = (2 * i, 2 * i + 1) if interleaved else (i, i + R // 2)
            c, s = np.float32(math.cos(ang)), np.float32(math.sin(ang))
            assert abs(out[t, i, j0] - c) <= 2.0 ** -24 and abs(out[t, i, j1] - s) <= 2.0 ** -24
            others = np.delete(out[t, i], [j0, j1])
            assert np.all(others == 0.0)


def test_roped_dot_product_depends_only_on_position_difference():
    # identical q and k vectors at every token of one long sequence
    D = R = 64
    n = 40
    case = _store_case(lengths=(n,), cache_lengths=(10,), num_pages=8, max_pages=4, P=16, Hq=1,
                       Hk=1, seed=21)
    case.buf[:] = case.buf[0]
    res = oracle.run_case(case)
    q = res.traces[0]["q_exact"][:, 0, :]          # [n, D], position 10 + t
    k = res.traces[0]["k_exact"][:, 0, :]
    scale = np.linalg.norm(q[0]) * np.linalg.norm(k[0])
    for delta in (0, 1, 5, 17):
        dots = np.array([q[t + delta] @ k[t] for t in range(n - delta)])
        assert np.all(np.abs(dots - dots[0]) <= 1e-6 * scale), delta
    # ... and it really varies with the difference
    assert abs(q[5] @ k[0] - q[0] @ k[0]) > 1e-3 * scale


def test_half_split_equals_permuted_interleaved():
    for R in (64, 32):
        hs = _store_case(interleaved=False, rope_dim=R, lengths=(9, 4), cache_lengths=(2, 40),
                         num_pages=8, max_pages=4, seed=13)
        il = _store_case(interleaved=True, rope_dim=R, lengths=(9, 4), cache_lengths=(2, 40),
                         num_pages=8, max_pages=4, seed=13)
        D, H = 64, 4 + 2 * 2
        perm = np.arange(D)
        perm[0:R:2] = np.arange(R // 2)             # interleaved slot 2i <- x[i]
        perm[1:R:2] = np.arange(R // 2) + R // 2    # interleaved slot 2i+1 <- x[i + R/2]
        x = hs.buf.reshape(hs.T, H, D)
        il.buf = np.ascontiguousarray(x[:, :, perm].reshape(hs.T, H * D))
        r_hs, r_il = oracle.run_case(hs), oracle.run_case(il)
        inv = np.argsort(perm)
        q_il = r_il.q_out[0].reshape(hs.T, 4, D)[:, :, inv].reshape(hs.T, 4 * D)
        assert np.array_equal(q_il, r_hs.q_out[0])
        k_il = r_il.pools[0][:, 0][..., inv]
        assert np.array_equal(k_il, r_hs.pools[0][:, 0])


def test_identity_page_table_is_a_dense_cache():
    # page_size >= every position: sequence b owns page b, so the pool's
    # K plane is a dense [batch, seq, head, dim] array
    lengths, clen = (5, 0, 12, 3), (4, 9, 0, 20)
    P = 32
    case = _store_case(lengths=lengths, cache_lengths=clen, P=P, num_pages=4, max_pages=1, seed=17)
    case.caches[0].lookup_table = np.arange(4, dtype=np.uint32).reshape(4, 1)
    res = oracle.run_case(case)
    dense_k = res.pools[0][:, 0, 0]                 # [b, pos, h, d]
    Hq, Hk, D = 4, 2, 64
    for t, b, cseq, pos in brute.walk_tokens(case):
        y, _ = brute.rope_complex(brute.as_f64(case.buf[t, Hq * D:(Hq + 1) * D], sc.F32),
                                  case.freqs[pos], 64, True)
        assert np.allclose(brute.as_f64(dense_k[b, pos, 0], sc.F32), y, rtol=0, atol=1e-6)
    # a permuted table moves whole pages, not values
    perm = np.array([2, 0, 3, 1], dtype=np.uint32)
    case2 = _store_case(lengths=lengths, cache_lengths=clen, P=P, num_pages=4, max_pages=1,
                        seed=17)
    case2.caches[0].lookup_table = perm.reshape(4, 1)
    res2 = oracle.run_case(case2)
    assert np.array_equal(res2.pools[0][perm], res.pools[0])


def test_copies_keep_every_bit_including_specials():
    for dtype in (sc.F32, sc.BF16, sc.F16):
        case = _store_case(dtype=dtype, rope_dim=32, lengths=(6, 9), cache_lengths=(1, 3),
                           specials=True, seed=23)
        res = oracle.run_case(case)
        tol = {sc.F32: 2.0 ** -23, sc.BF16: 2.0 ** -8, sc.F16: 2.0 ** -11}[dtype]
        written = _check_store_against_brute(case, res, pair_tol=tol)
        _check_sentinels(case, res.pools[0], written)


def test_empty_batch_writes_nothing():
    case = _store_case(lengths=(0, 0), cache_lengths=(0, 4), seed=2)
    res = oracle.run_case(case)
    assert res.status == 0 and case.T == 0
    assert np.all(res.pools[0] == sc.SENTINEL[sc.F32])


def test_out_of_range_position_is_an_error():
    case = _store_case(lengths=(3, 5), cache_lengths=(0, 60), max_pages=5, num_pages=12,
                       seed=2)                                            # 60 + 4 >= 64
    assert oracle.run_case(case).status == -6


# --------------------------------------------------------------------------
# RMSNorm
# --------------------------------------------------------------------------

def _norm_case(D=64, R=64, lengths=(4,), clen=(0,), eps=1e-6, w=0.0, mbc=True, dtype=sc.F32,
               k_in_cache=False, seed=31, Hq=2, Hk=1, interleaved=True):
    return sc.make_norm_case("pin_norm", seed, dtype, list(lengths), list(clen), Hq=Hq, Hk=Hk,
                             D=D, rope_dim=R, interleaved=interleaved, theta=1e4,
                             max_seq_len=64, P=16, L=1, layer=0, k_in_cache=k_in_cache, eps=eps,
                             weight_offset=w, multiply_before_cast=mbc)


def test_rmsnorm_constant_vector_closed_form():
    # x = c * ones at position 0 (rope is the identity there):
    # y_j = c / sqrt(c^2 + eps) * (gamma_j + w)
    D = 64
    for c, eps, w in ((0.75, 1e-6, 0.0), (3e-3, 1e-5, 0.5), (-2.0, 0.25, -0.25)):
        case = _norm_case(lengths=(1,), clen=(0,), eps=eps, w=w, D=D)
        case.buf[:] = sc.to_bits(np.full(case.buf.shape, c), sc.F32)
        res = oracle.run_case(case)
        g = brute.as_f64(case.bands[0].q_gamma, sc.F32)
        eps32 = float(np.float32(eps))
        w32 = float(np.float32(w))
        want = c / math.sqrt(c * c + eps32) * (g + w32)
        got = brute.as_f64(res.q_out[0][0, :D], sc.F32)
        assert np.all(np.abs(got - want) <= 2.0 ** -23 * np.abs(want) + 1e-30)


def test_rmsnorm_invariants():
    D = 64
    case = _norm_case(lengths=(3,), clen=(0,), eps=0.0)
    case.bands[0].q_gamma = sc.to_bits(np.ones(D), sc.F32)
    r1 = oracle.run_case(case)
    y = r1.traces[0]["q_exact"][0]                  # position 0: no rotation
    # unit mean square with gamma = 1, eps = 0
    assert np.allclose((y ** 2).mean(axis=-1), 1.0, rtol=1e-12)
    # scale invariance: x -> 4x gives the same output (powers of two are exact)
    x = brute.as_f64(case.buf, sc.F32)
    case.buf = sc.to_bits(4.0 * x, sc.F32)
    r2 = oracle.run_case(case)
    assert np.array_equal(r1.q_out[0], r2.q_out[0])
    # gamma = 0, w = 1  ==  gamma = 1, w = 0
    case.bands[0].q_gamma = sc.to_bits(np.zeros(D), sc.F32)
    case.weight_offset = 1.0
    r3 = oracle.run_case(case)
    assert np.array_equal(r3.q_out[0], r2.q_out[0])


def test_rmsnorm_epsilon_sits_inside_the_root():
    # with x = c*1 and c^2 = eps, 1/sqrt(c^2 + eps) = 1/(c*sqrt 2)
    c = 2.0 ** -4
    case = _norm_case(lengths=(1,), eps=c * c, D=64)
    case.bands[0].q_gamma = sc.to_bits(np.ones(64), sc.F32)
    case.buf[:] = sc.to_bits(np.full(case.buf.shape, c), sc.F32)
    y = oracle.run_case(case).traces[0]["q_exact"][0, 0]
    assert np.allclose(y, 1.0 / math.sqrt(2.0), rtol=1e-7)


def test_norm_then_rope_order_and_k_paths():
    # K from the buffer and K in the cache give the same K row when the cache
    # holds what the buffer holds; V copied only on the buffer path
    case_buf = _norm_case(lengths=(5, 3), clen=(2, 0), Hk=2, seed=41)
    case_cache = _norm_case(lengths=(5, 3), clen=(2, 0), Hk=2, seed=41, k_in_cache=True)
    # put the buffer's K values into the cache rows
    cache = case_cache.caches[0]
    Hq, Hk, D = 2, 2, 64
    cache.prefill = []
    pages, slots, vals = [], [], []
    for t, b, cseq, pos in brute.walk_tokens(case_cache):
        page, slot = brute.page_slot(cache, cseq, pos)
        pages.append(page)
        slots.append(slot)
        vals.append(case_buf.buf[t, Hq * D:(Hq + Hk) * D].reshape(Hk, D))
    n = len(pages)
    cache.prefill.append((np.array(pages), np.zeros(n, np.int64), np.zeros(n, np.int64),
                          np.array(slots), np.array(vals)))
    case_cache.buf = case_buf.buf.copy()
    r_buf, r_cache = oracle.run_case(case_buf), oracle.run_case(case_cache)
    assert np.array_equal(r_buf.pools[0][:, 0], r_cache.pools[0][:, 0])
    assert np.array_equal(r_buf.q_out[0], r_cache.q_out[0])
    assert np.all(r_cache.pools[0][:, 1] == sc.SENTINEL[sc.F32])
    # norm precedes rope: rope(norm(x)) differs from norm(rope(x)) when gamma varies
    x = brute.as_f64(case_buf.buf[3, :D], sc.F32)
    pos = 2 + 3
    g = brute.as_f64(case_buf.bands[0].q_gamma, sc.F32)
    rot_then_norm, _ = brute.rope_complex(x, case_buf.freqs[pos], 64, True)
    rot_then_norm = rot_then_norm / math.sqrt((rot_then_norm ** 2).mean() + 1e-6) * g
    got = r_buf.traces[0]["q_exact"][3, 0]
    assert not np.allclose(got, rot_then_norm, rtol=1e-4)


# --------------------------------------------------------------------------
# radd
# --------------------------------------------------------------------------

def _radd_case(seed=51, dtype=sc.BF16, lengths=(3, 0, 7, 2), clen=(5, 1, 9, 0, 30, 2),
               boff=2, a_values=None):
    return sc.make_radd_case("pin_radd", seed, dtype, list(lengths), list(clen), boff, Hk=2, D=64,
                             P=8, L=2, layer=1, a_values=a_values)


@pytest.mark.parametrize("dtype", [sc.F32, sc.BF16, sc.F16])
def test_radd_is_one_binary32_add_per_element(dtype):
    case = _radd_case(dtype=dtype)
    # sprinkle subnormals, zeros of both signs and large values into a
    a = case.buf.copy()
    specials = (sc._special_values(dtype))
    finite = specials[np.isfinite(brute.as_f64(specials, dtype))]
    flat = a.reshape(-1)
    flat[::7] = finite[np.arange(len(flat[::7])) % len(finite)]
    case.buf = a
    before = case.caches[0].materialize()
    res = oracle.run_case(case)
    cache = case.caches[0]
    Hk, D = 2, 64
    written = set()
    for t, b, cseq, pos in brute.walk_tokens(case):
        page, slot = brute.page_slot(cache, cseq, pos)
        for plane in (0, 1):
            for h in range(Hk):
                cur = before[page, plane, 1, slot, h]
                add = case.buf[t, plane * Hk * D + h * D: plane * Hk * D + (h + 1) * D]
                s32 = (brute.as_f64(cur, dtype).astype(np.float32) +
                       brute.as_f64(add, dtype).astype(np.float32))
                want = sc.to_bits(s32.astype(np.float64), dtype)
                assert np.array_equal(res.pools[0][page, plane, 1, slot, h], want), (t, plane, h)
                written.add((page, plane, 1, slot, h))
    mask = np.ones(before.shape[:5], dtype=bool)
    for w in written:
        mask[w] = False
    assert np.array_equal(res.pools[0][mask], before[mask])


def test_radd_of_zeros_changes_nothing():
    case = _radd_case()
    before = case.caches[0].materialize()
    case.buf = np.zeros_like(case.buf)                      # +0
    assert np.array_equal(oracle.run_case(case).pools[0], before)
    case.buf = np.full_like(case.buf, 0x8000)               # -0: x + (-0) == x for every x
    assert np.array_equal(oracle.run_case(case).pools[0], before)

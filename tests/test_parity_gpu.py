"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle.

Every case runs on seeded synthetic inputs shaped like the five workloads
(tiny fp32; Llama-3-8B prefill and decode; dual-band RMSNorm + RoPE; radd),
at reduced sizes that still span many waves and a ragged tail, at full size,
in a long-context prefill that reaches the last freqs row,
and on edge cases (empty batch and sequences, page size 1, head_dim 64/256,
fp32 and bf16, partial rope in both layouts, padded strides, special values,
multiply_before_cast = false, K from the buffer or in the cache).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from synth import cases as sc  # noqa: E402
from synth import prng  # noqa: E402


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests import gpu_harness as gh
    from tests import parity
    return gh, parity


def run_and_compare(case, ulps=1):
    gh, parity = _gpu()
    print(f"[parity] {case.name} op={case.op} dtype={case.dtype} T={case.T} seed={case.seed}",
          flush=True)
    res = oracle.run_case(case)
    dc = gh.upload(case)
    gh.run(dc)
    torch.cuda.synchronize()
    rep = parity.compare(case, dc, res, ulps=ulps)
    print(f"[parity] {case.name} ok {dict(rep)}", flush=True)
    return rep


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------

def test_tiny_fp32():
    run_and_compare(sc.tiny_fp32())


@pytest.mark.parametrize("workload", ["prefill", "decode", "dual", "radd", "prefill_tp8", "decode_tp8", "dual_tp8"])
@pytest.mark.parametrize("seed", [None, 101])
def test_small_workloads(workload, seed):
    kw = {} if seed is None else {"seed": seed}
    run_and_compare(sc.WORKLOADS[workload](small=True, **kw))


@pytest.mark.parametrize("workload", ["prefill", "decode", "dual", "radd", "prefill_tp8", "decode_tp8", "dual_tp8"])
def test_full_size_workloads(workload):
    run_and_compare(sc.WORKLOADS[workload]())


@pytest.mark.parametrize("cache_dtype", [None, sc.FP8])
def test_long_context_prefill_to_the_table_end(cache_dtype):
    # Llama-3-8B heads over sequences that reach the last freqs row: one of
    # 8192 new tokens (positions 0..8191), one continuing a 4096-row cache to
    # 8191, and two long ragged ones -- about 27k tokens, several generations
    # of waves per SIMD and three times the prefill workload's batch
    lens = np.array([8192, 4096, 7999, 7001], np.int64)
    clen = np.array([0, 4096, 192, 0], np.int64)
    run_and_compare(sc.make_store_case("long_context", 41, sc.BF16, lens, clen, Hq=32, Hk=8,
                                       D=128, rope_dim=128, interleaved=False, theta=5e5,
                                       max_seq_len=8192, P=128, L=4, layer=2,
                                       cache_dtype=cache_dtype))


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------

def _store(name, seed, dtype, lengths, clen, D=128, R=None, il=True, Hq=8, Hk=2, P=16, L=2,
           layer=1, msl=512, **kw):
    R = R or D
    return sc.make_store_case(name, seed, dtype, lengths, clen, Hq=Hq, Hk=Hk, D=D, rope_dim=R,
                              interleaved=il, theta=1e4, max_seq_len=msl, P=P, L=L, layer=layer,
                              **kw)


@pytest.mark.parametrize("dtype", [sc.F32, sc.BF16, sc.F16])
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("il", [True, False])
def test_store_head_dims_and_layouts(dtype, D, il):
    lens = [5, 0, 17, 1, 33, 0, 2]
    clen = [0, 3, 40, 9, 100, 7, 250]
    run_and_compare(_store(f"store_{dtype}_{D}_{il}", 7, dtype, lens, clen, D=D, il=il))


@pytest.mark.parametrize("dtype", [sc.F32, sc.BF16, sc.F16])
@pytest.mark.parametrize("il", [True, False])
def test_store_partial_rope_padding_and_specials(dtype, il):
    R = 16 if dtype == sc.F32 else 32
    case = _store("store_partial", 8, dtype, [9, 4, 21], [2, 60, 7], D=128, R=R, il=il,
                  specials=True, q_out_pad=16, row_pad=24)
    run_and_compare(case)


def test_store_page_size_one_and_odd_page_size():
    run_and_compare(_store("page1", 9, sc.BF16, [3, 7, 2], [5, 0, 11], P=1, msl=64))
    run_and_compare(_store("page24", 10, sc.BF16, [30, 17], [5, 40], P=24, msl=128))


def test_store_empty_batch_is_a_no_op():
    gh, parity = _gpu()
    case = _store("empty", 11, sc.BF16, [0, 0, 0], [4, 0, 9])
    assert case.T == 0
    run_and_compare(case)


def test_store_single_token_and_last_position():
    run_and_compare(_store("last_pos", 12, sc.BF16, [1], [511], msl=512, P=16))


def test_store_many_tiny_sequences():
    lens = prng.integers(13, 1, 700, 0, 3)
    clen = prng.integers(13, 2, 700, 0, 200)
    run_and_compare(_store("tiny_seqs", 13, sc.BF16, lens, clen, Hq=4, Hk=1, P=8, msl=256))


def _norm(name, seed, dtype, lengths, clen, k_in_cache, D=128, R=64, il=True, **kw):
    return sc.make_norm_case(name, seed, dtype, lengths, clen, Hq=6, Hk=2, D=D, rope_dim=R,
                             interleaved=il, theta=1e4, max_seq_len=512, P=32, L=2, layer=1,
                             k_in_cache=k_in_cache, **kw)


@pytest.mark.parametrize("dtype", [sc.F32, sc.BF16, sc.F16])
@pytest.mark.parametrize("k_in_cache", [False, True])
@pytest.mark.parametrize("il", [True, False])
def test_norm_single_band(dtype, k_in_cache, il):
    case = _norm("norm", 14, dtype, [7, 0, 30, 3], [0, 5, 17, 200], k_in_cache, il=il,
                 weight_offset=0.0 if dtype == sc.F32 else 0.25, eps=1e-5)
    run_and_compare(case)


@pytest.mark.parametrize("q_norm,k_norm", [(True, False), (False, True), (False, False)])
def test_norm_on_one_role_only(q_norm, k_norm):
    case = _norm("norm_roles", 15, sc.BF16, [11, 5], [3, 0], True, q_norm=q_norm, k_norm=k_norm)
    run_and_compare(case)


@pytest.mark.parametrize("dtype", [sc.BF16, sc.F16])
def test_norm_multiply_after_cast(dtype):
    case = _norm("norm_mbc0", 16, dtype, [25, 9], [0, 31], False, multiply_before_cast=False,
                 weight_offset=0.5)
    run_and_compare(case)


def test_norm_head_dim_64_and_256():
    run_and_compare(_norm("norm64", 17, sc.BF16, [12, 3], [1, 2], True, D=64, R=64))
    run_and_compare(_norm("norm256", 18, sc.BF16, [12, 3], [1, 2], False, D=256, R=128))


def test_dual_band_small_with_distinct_eps_and_nonzero_cache_lengths():
    case = sc.make_dual_case("dual_eps", 19, sc.BF16, [5, 0, 40, 9], Hq_main=16, Hk_main=4,
                             Hq_index=4, D=128, rope_dim=64, interleaved=False, theta=1e4,
                             max_seq_len=1024, P_main=32, P_index=16, eps_main=1e-6,
                             eps_index=1e-3, weight_offset=0.125, cache_lengths=[3, 0, 100, 7])
    run_and_compare(case)


@pytest.mark.parametrize("cache_dtype", [None, sc.FP8])
@pytest.mark.parametrize("mbc", [True, False])
@pytest.mark.parametrize("batch", [5, 40])
def test_dual_band_index_cache_has_its_own_lengths(cache_dtype, mbc, batch):
    # the index cache's lengths differ from the main cache's, so its rows sit
    # at other positions (another freqs row) than the main band's; 5
    # sequences take the small-batch lookup, 40 the guessed one
    lens = prng.integers(27, 1, batch, 0, 12)
    clm = prng.integers(27, 2, batch, 0, 900)
    cli = prng.integers(27, 3, batch, 0, 900)
    case = sc.make_dual_case(f"dual_own_lengths_{batch}", 27, sc.BF16, lens, Hq_main=16,
                             Hk_main=4, Hq_index=4, D=128, rope_dim=64, interleaved=bool(batch % 2),
                             theta=1e4, max_seq_len=1024, P_main=32, P_index=16, eps_main=1e-6,
                             eps_index=1e-2, weight_offset=0.25, multiply_before_cast=mbc,
                             cache_lengths=clm, index_cache_lengths=cli,
                             main_cache_dtype=cache_dtype, index_cache_dtype=cache_dtype)
    run_and_compare(case)


@pytest.mark.parametrize("cache_dtype", [None, sc.FP8])
def test_norm_multiply_after_cast_k_in_cache(cache_dtype):
    case = _norm("norm_mbc0_inplace", 28, sc.BF16, [19, 3, 0, 40], [0, 7, 2, 100], True,
                 multiply_before_cast=False, weight_offset=0.5, cache_dtype=cache_dtype)
    run_and_compare(case)


def test_radd_fp32_and_subnormals():
    case = sc.make_radd_case("radd_f32", 20, sc.F32, [4, 0, 13, 7], [3, 9, 1, 0, 30, 2, 5], 2,
                             Hk=3, D=64, P=8, L=2, layer=1)
    run_and_compare(case)
    # bf16 subnormals, zeros and extremes in a
    case = sc.make_radd_case("radd_sub", 21, sc.BF16, [6, 9], [1, 2, 3], 1, Hk=2, D=128, P=16,
                             L=1, layer=0)
    specials = np.array([0x0000, 0x8000, 0x0001, 0x807F, 0x0080, 0x7F7F, 0x3C00], np.uint16)
    flat = case.buf.reshape(-1)
    flat[::3] = specials[np.arange(len(flat[::3])) % len(specials)]
    run_and_compare(case)


def test_radd_f16_specials():
    case = sc.make_radd_case("radd_f16", 22, sc.F16, [5, 11, 0, 3], [4, 1, 0, 9, 2], 1, Hk=2,
                             D=128, P=16, L=2, layer=1)
    specials = np.array([0x0000, 0x8000, 0x0001, 0x83FF, 0x0400, 0x7BFF, 0xFBFF, 0x3C00],
                        np.uint16)
    flat = case.buf.reshape(-1)
    flat[::5] = specials[np.arange(len(flat[::5])) % len(specials)]
    run_and_compare(case)


# ---------------------------------------------------------------------------
# bf16 freqs_cis tables (the table's dtype is its own parameter)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [sc.F32, sc.BF16, sc.F16])
@pytest.mark.parametrize("il", [True, False])
def test_store_bf16_freqs(dtype, il):
    R = 64 if il else 128
    case = _store(f"store_bf16freqs_{dtype}_{il}", 23, dtype, [9, 1, 26, 0, 4], [0, 70, 3, 8, 300],
                  D=128, R=R, il=il, freq_dtype=sc.BF16)
    run_and_compare(case)


@pytest.mark.parametrize("dtype", [sc.F32, sc.BF16, sc.F16])
@pytest.mark.parametrize("il", [True, False])
def test_norm_bf16_freqs(dtype, il):
    case = _norm(f"norm_bf16freqs_{dtype}_{il}", 24, dtype, [13, 2, 0, 21], [1, 0, 44, 250],
                 il ^ (dtype == sc.F16), il=il, freq_dtype=sc.BF16, weight_offset=0.0)
    run_and_compare(case)


def test_dual_band_bf16_freqs_f16():
    case = sc.make_dual_case("dual_f16_bf16freqs", 25, sc.F16, [6, 0, 31, 2], Hq_main=16,
                             Hk_main=4, Hq_index=4, D=128, rope_dim=64, interleaved=True,
                             theta=1e4, max_seq_len=512, P_main=32, P_index=16, eps_main=1e-6,
                             eps_index=1e-5, weight_offset=0.0, cache_lengths=[0, 3, 17, 400],
                             freq_dtype=sc.BF16)
    run_and_compare(case)


# ---------------------------------------------------------------------------
# trailing-dims partial rope (rope_tail)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [sc.F32, sc.BF16, sc.F16])
@pytest.mark.parametrize("il", [True, False])
@pytest.mark.parametrize("D,R", [(128, 64), (128, 32), (256, 64), (64, 32)])
def test_store_trailing_partial_rope(dtype, il, D, R):
    if dtype == sc.F32 and R == 32 and D == 64:
        R = 16
    run_and_compare(_store(f"tail_{dtype}_{il}_{D}_{R}", 70, dtype, [7, 0, 19, 3], [2, 9, 40, 0],
                           D=D, R=R, il=il, rope_tail=True))


@pytest.mark.parametrize("k_in_cache", [False, True])
@pytest.mark.parametrize("il", [True, False])
def test_norm_trailing_partial_rope(k_in_cache, il):
    run_and_compare(_norm("norm_tail", 71, sc.BF16, [9, 4, 0, 17], [1, 0, 30, 5], k_in_cache,
                          il=il, R=32, rope_tail=True, weight_offset=0.25))


def test_dual_band_trailing_partial_rope():
    case = sc.make_dual_case("dual_tail", 72, sc.BF16, [5, 0, 21, 8], Hq_main=16, Hk_main=4,
                             Hq_index=4, D=128, rope_dim=64, interleaved=True, theta=1e4,
                             max_seq_len=512, P_main=32, P_index=16, cache_lengths=[0, 3, 17, 400],
                             rope_tail=True)
    run_and_compare(case)


def test_bshd_and_fp8_trailing_partial_rope():
    run_and_compare(sc.make_bshd_case("bshd_tail", 73, sc.BF16, [5, 0, 17, 30], 24, [0, 9, 100, 3],
                                      Hq=6, Hk=2, D=128, rope_dim=64, interleaved=False,
                                      theta=1e4, max_seq_len=512, capacity=512, L=2, layer=1,
                                      rope_tail=True))
    run_and_compare(_store("fp8_tail", 74, sc.BF16, [6, 13, 2], [0, 5, 77], D=128, R=64, il=True,
                           rope_tail=True, cache_dtype=sc.FP8))

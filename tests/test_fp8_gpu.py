"""GPU parity of FP8 (OCP E4M3) caches and of Q outputs in another dtype
against the CPU oracle (rope_split_store_paged_ragged page, Parameters:
q_out_dtype; Args: kv_collection with a scale dtype and a quantization
granularity; fused_dual_qk_rms_norm_rope_ragged_paged page, signature: cache
dtypes of their own).

Roped K rows are compared value by value within one E4M3 step; V rows,
radd rows, every untouched code and every scale outside the roped rows must
match bit for bit.  Cases: every op (store, single-band norm with K from the
buffer and in place, dual band, radd, padded grid), every input dtype, both
layouts, f32 and bf16 scales, head_dim 64 / 128 / 256, the workloads at
reduced and full size, every Q output dtype pair over plain and FP8 caches,
the dual band with one plain and one FP8 cache (either way round), and
bit-identical results across launch configurations (XCD remap on and off).
"""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from synth import cases as sc  # noqa: E402


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests import gpu_harness as gh
    from tests import parity
    return gh, parity


def run_and_compare(case, ulps=1):
    gh, parity = _gpu()
    print(f"[fp8] {case.name} op={case.op} dtype={case.dtype} q={case.q_dtype} "
          f"cache={[c.dtype for c in case.caches]} T={case.T} seed={case.seed}", flush=True)
    res = oracle.run_case(case)
    dc = gh.upload(case)
    gh.run(dc)
    torch.cuda.synchronize()
    rep = parity.compare(case, dc, res, ulps=ulps)
    print(f"[fp8] {case.name} ok {dict(rep)}", flush=True)
    return rep


def _store(name, seed, dtype, D=128, R=None, il=True, scale=sc.F32, cache=sc.FP8, q_out=None,
           lens=(5, 0, 17, 1, 33, 2), clen=(0, 3, 40, 9, 100, 250)):
    return sc.make_store_case(name, seed, dtype, list(lens), list(clen), Hq=8, Hk=2, D=D,
                              rope_dim=R or D, interleaved=il, theta=1e4, max_seq_len=512, P=16,
                              L=2, layer=1, cache_dtype=cache, scale_dtype=scale,
                              q_out_dtype=q_out)


@pytest.mark.parametrize("workload", ["prefill_fp8", "decode_fp8", "dual_fp8", "radd_fp8",
                                      "bshd_fp8"])
def test_fp8_small_workloads(workload):
    run_and_compare(sc.WORKLOADS[workload](small=True))


@pytest.mark.parametrize("workload", ["prefill_fp8", "decode_fp8"])
def test_fp8_full_size_store_workloads(workload):
    run_and_compare(sc.WORKLOADS[workload]())


@pytest.mark.parametrize("scale", [sc.F32, sc.BF16])
@pytest.mark.parametrize("il", [True, False])
@pytest.mark.parametrize("dtype", [sc.F32, sc.BF16, sc.F16])
def test_fp8_store_dtypes_layouts_scales(dtype, il, scale):
    run_and_compare(_store(f"fp8_store_{dtype}_{il}_{scale}", 60, dtype, il=il, scale=scale))


@pytest.mark.parametrize("D", [64, 256])
def test_fp8_store_head_dims_and_partial_rope(D):
    run_and_compare(_store(f"fp8_store_D{D}", 61, sc.BF16, D=D, R=D // 2, il=False))


@pytest.mark.parametrize("k_in_cache", [False, True])
@pytest.mark.parametrize("scale", [sc.F32, sc.BF16])
@pytest.mark.parametrize("dtype", [sc.BF16, sc.F16, sc.F32])
def test_fp8_norm_single_band(dtype, scale, k_in_cache):
    case = sc.make_norm_case(f"fp8_norm_{dtype}_{scale}_{k_in_cache}", 62, dtype, [7, 0, 30, 3],
                             [0, 5, 17, 200], Hq=6, Hk=2, D=128, rope_dim=64, interleaved=True,
                             theta=1e4, max_seq_len=512, P=32, L=2, layer=1, k_in_cache=k_in_cache,
                             weight_offset=0.0, cache_dtype=sc.FP8, scale_dtype=scale)
    run_and_compare(case)


def test_fp8_dual_band_half_split():
    case = sc.make_dual_case("fp8_dual", 63, sc.BF16, [5, 0, 40, 9], Hq_main=16, Hk_main=4,
                             Hq_index=4, D=128, rope_dim=64, interleaved=False, theta=1e4,
                             max_seq_len=1024, P_main=32, P_index=16, eps_main=1e-6,
                             eps_index=1e-3, cache_lengths=[3, 0, 100, 7],
                             main_cache_dtype=sc.FP8, index_cache_dtype=sc.FP8,
                             scale_dtype=sc.BF16)
    run_and_compare(case)


@pytest.mark.parametrize("scale", [sc.F32, sc.BF16])
@pytest.mark.parametrize("dtype", [sc.BF16, sc.F32, sc.F16])
def test_fp8_radd_bit_exact(dtype, scale):
    case = sc.make_radd_case(f"fp8_radd_{dtype}_{scale}", 64, dtype, [4, 0, 13, 7],
                             [3, 9, 1, 0, 30, 2, 5], 2, Hk=3, D=64, P=8, L=2, layer=1,
                             a_std=0.05, cache_dtype=sc.FP8, scale_dtype=scale)
    run_and_compare(case)


def test_fp8_bshd_padded_grid():
    case = sc.make_bshd_case("fp8_bshd", 65, sc.BF16, [5, 0, 17, 30, 2], 24, [0, 9, 100, 3, 480],
                             Hq=6, Hk=2, D=128, rope_dim=128, interleaved=True, theta=1e4,
                             max_seq_len=512, capacity=512, L=2, layer=1, cache_dtype=sc.FP8)
    run_and_compare(case)


@pytest.mark.parametrize("cache", [None, sc.FP8])
@pytest.mark.parametrize("dtype,q_out", [(sc.BF16, sc.F32), (sc.F16, sc.F32), (sc.F32, sc.BF16),
                                         (sc.F32, sc.F16), (sc.BF16, sc.F16), (sc.F16, sc.BF16)])
def test_q_output_dtype(dtype, q_out, cache):
    for il in (True, False):
        R = 32 if il else 64
        run_and_compare(_store(f"qout_{dtype}_{q_out}_{cache}_{il}", 66, dtype, R=R, il=il,
                               cache=cache, q_out=q_out))


def _mixed_dual(main, index, small=True, seed=4):
    """The dual-band workload's shapes (64 Q-main, 8 KV, 16 Q-index heads,
    head_dim 128, partial rope 64) with the two caches of different types."""
    B = 4 if small else 16
    from synth import prng
    lens = prng.integers(seed, sc.S_LENS, B, 1, 150 if small else 1024)
    return sc.make_dual_case(f"dual_mixed_{main}_{index}_{'small' if small else 'full'}", seed,
                             sc.BF16, lens, Hq_main=64, Hk_main=8, Hq_index=16, D=128,
                             rope_dim=64, interleaved=True, theta=1e4, max_seq_len=8192,
                             P_main=64, P_index=64, main_cache_dtype=main,
                             index_cache_dtype=index)


@pytest.mark.parametrize("small", [True, False])
@pytest.mark.parametrize("main,index", [(sc.BF16, sc.FP8), (sc.FP8, sc.BF16)])
def test_fp8_dual_band_mixed_cache_dtypes(main, index, small):
    # fused_dual_qk_rms_norm_rope_ragged_paged page, Signature: the two
    # caches' element types are separate parameters
    run_and_compare(_mixed_dual(main, index, small))


@pytest.mark.parametrize("main,index", [(sc.F16, sc.FP8), (sc.FP8, sc.F16)])
def test_fp8_dual_band_mixed_half_split_bf16_scales_own_lengths(main, index):
    case = sc.make_dual_case("fp8_dual_mixed_hs", 64, sc.F16, [5, 0, 40, 9, 17], Hq_main=16,
                             Hk_main=4, Hq_index=4, D=128, rope_dim=64, interleaved=False,
                             theta=1e4, max_seq_len=1024, P_main=32, P_index=16, eps_main=1e-6,
                             eps_index=1e-3, weight_offset=0.25, multiply_before_cast=False,
                             cache_lengths=[3, 0, 100, 7, 500],
                             index_cache_lengths=[0, 9, 33, 200, 1], main_cache_dtype=main,
                             index_cache_dtype=index, scale_dtype=sc.BF16)
    run_and_compare(case)


def test_fp8_dual_band_mixed_launch_configuration_does_not_change_bits():
    gh, _ = _gpu()
    case = _mixed_dual(sc.BF16, sc.FP8)
    ref = None
    for remap, ppw, wpb in [(r, p, w) for r in ("0", "1", "2") for p in ("0", "1", "2", "3")
                            for w in ("0", "1", "4")]:
        dc = gh.upload(case)
        with gh.knobs(remap, ppw, wpb, pack=1):      # packing is not used for mixed pairs
            gh.run(dc)
        torch.cuda.synchronize()
        snap = [gh.to_numpy_bits(q, case.q_dtype) for q in dc.q_out]
        snap += [gh.to_numpy_bits(c.pool, c.host.dtype) for c in dc.caches]
        snap += [gh.to_numpy_bits(c.scales, c.host.scale_dtype) for c in dc.caches
                 if c.scales is not None]
        if ref is None:
            ref = snap
        else:
            for i, (x, y) in enumerate(zip(ref, snap)):
                assert np.array_equal(x, y), f"mixed dual remap={remap} ppw={ppw} wpb={wpb}: buffer {i}"


@pytest.mark.parametrize("workload", ["prefill_fp8", "radd_fp8", "dual_fp8"])
def test_fp8_launch_configuration_does_not_change_bits(workload, monkeypatch):
    gh, _ = _gpu()
    case = sc.WORKLOADS[workload](small=True)
    ref = None
    for remap, ppw, wpb in [(r, p, w) for r in ("0", "1", "2") for p in ("0", "1", "3")
                            for w in ("0", "1", "4")]:
        dc = gh.upload(case)
        with gh.knobs(remap, ppw, wpb):
            gh.run(dc)
        torch.cuda.synchronize()
        snap = [gh.to_numpy_bits(q, case.q_dtype) for q in dc.q_out]
        snap += [gh.to_numpy_bits(c.pool, c.host.dtype) for c in dc.caches]
        snap += [gh.to_numpy_bits(c.scales, c.host.scale_dtype) for c in dc.caches]
        if ref is None:
            ref = snap
        else:
            for i, (x, y) in enumerate(zip(ref, snap)):
                assert np.array_equal(x, y), f"{workload} remap={remap} ppw={ppw} wpb={wpb}: buffer {i}"

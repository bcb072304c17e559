"""matmul_fused_partial_rmsnorm_noalloc (the GEMV + partial RMSNorm with the
library's own scratch, for callers that cannot allocate) against the
workspace entry point, through the C ABI.

Both run the same kernel, so their outputs must be the same bits; the first
call of each pair is also checked against the CPU oracle with the GEMV's
parity bar.  The calls come in a row on one GPU: a large one, then a smaller
one (fewer rows and normed columns), then the largest the scratch holds, then
nothing normed, then the bench shape again -- each call relies on the
previous one having left the shared counter at zero.  Sizes past the scratch
return QRP_EINVAL before anything is launched.
"""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from synth import cases as sc  # noqa: E402

SCRATCH_VALUES = 131072        # m * n_normed the library's scratch holds


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import qk_rope_paged_amd as qrp
    from tests import gemv_parity
    from tests import gpu_harness as gh
    return qrp, gh, gemv_parity


def _noalloc(qrp, gh, dg, raise_on_error=True):
    c = dg.case
    return qrp.matmul_fused_partial_rmsnorm_noalloc(
        dg.normed if c.n_normed else None, c.normed_row_stride,
        dg.unnormed if c.n_normed < c.n else None, c.unnormed_row_stride,
        dg.x, c.x.shape[1], c.m, dg.w, c.w.shape[1], c.n, c.k, dg.gamma, c.n_normed,
        c.epsilon, c.weight_offset, gh.QRP_DT[c.dtype],
        transpose_b=int(getattr(c, "transpose_b", 1)), raise_on_error=raise_on_error)


def _pair(case, check_oracle):
    qrp, gh, gp = _gpu()
    print(f"[noalloc] {case.name} dtype={case.dtype} m={case.m} k={case.k} n={case.n} "
          f"n_normed={case.n_normed}", flush=True)
    ref = gh.upload_gemv(case)
    gh.run_gemv(ref)
    mine = gh.upload_gemv(case)
    _noalloc(qrp, gh, mine)
    torch.cuda.synchronize()
    for a, b, what in ((ref.normed, mine.normed, "normed"),
                       (ref.unnormed, mine.unnormed, "unnormed")):
        ga, gb = gh.to_numpy_bits(a, case.dtype), gh.to_numpy_bits(b, case.dtype)
        assert np.array_equal(ga, gb), f"{case.name}: {what} differs from the workspace call"
    if check_oracle:
        res = oracle.run_gemv(case)
        assert res.status == 0
        gp.check(case, res, gh.to_numpy_bits(mine.normed, case.dtype),
                 gh.to_numpy_bits(mine.unnormed, case.dtype))
    print(f"[noalloc] {case.name} ok", flush=True)


def test_noalloc_matches_the_workspace_call_on_calls_in_a_row():
    # large, then smaller, then the scratch's limit, then nothing normed, then again
    _pair(sc.make_gemv_case("noalloc_big", 81, sc.BF16, 4, 1024, 3000, 2500), True)
    _pair(sc.make_gemv_case("noalloc_small", 82, sc.BF16, 1, 512, 300, 100), True)
    _pair(sc.make_gemv_case("noalloc_limit", 83, sc.F16, 8, 256, 16400,
                            SCRATCH_VALUES // 8), False)
    _pair(sc.make_gemv_case("noalloc_unnormed", 84, sc.F32, 2, 256, 500, 0), True)
    _pair(sc.gemv_norm(small=True), True)


def test_noalloc_w_stored_k_by_n_on_calls_in_a_row():
    # W stored [k][n]: the slices' sums and the tiles' counters live in the
    # scratch too -- a split call, a smaller one, nothing normed, eight rows
    _pair(sc.make_gemv_case("noalloc_t_big", 87, sc.BF16, 4, 8192, 1000, 700,
                            transpose_b=False), True)
    _pair(sc.make_gemv_case("noalloc_t_small", 88, sc.F32, 1, 512, 100, 60,
                            transpose_b=False), True)
    _pair(sc.make_gemv_case("noalloc_t_unnormed", 89, sc.F16, 2, 4096, 64, 0,
                            transpose_b=False), True)
    _pair(sc.make_gemv_case("noalloc_t_rows8", 90, sc.BF16, 8, 2048, 200, 130,
                            transpose_b=False), True)
    _pair(sc.gemv_norm(small=True, transpose_b=False), True)


def test_noalloc_rejects_sizes_past_its_scratch():
    qrp, gh, _ = _gpu()
    case = sc.make_gemv_case("noalloc_over", 85, sc.BF16, 2, 64, 65600,
                             SCRATCH_VALUES // 2 + 1)
    dg = gh.upload_gemv(case)
    st = _noalloc(qrp, gh, dg, raise_on_error=False)
    assert st == qrp.QRP_EINVAL
    assert "scratch" in qrp.last_error()
    torch.cuda.synchronize()
    assert np.all(gh.to_numpy_bits(dg.normed, case.dtype) == sc.SENTINEL[case.dtype])
    # the limit itself still runs
    _pair(sc.make_gemv_case("noalloc_at_limit", 86, sc.BF16, 2, 64, 65600,
                            SCRATCH_VALUES // 2), False)

"""GPU parity of the fused GEMV + partial RMSNorm (MatmulFusedPartialRMSNorm
page) through the C ABI, against the CPU oracle, with the bar that
tests/gemv_parity.py derives from the kernel's binary32 arithmetic.

Cases: the bench shape (hidden 7168 -> 1536 normed + 576 passed through) at
full and reduced size; every dtype with 1, 2, 3, 5 and 8 input rows, padded
strides, a k that leaves a ragged last chunk round, and a norm boundary that
splits a wave's columns; nothing normed (no workspace at all), everything
normed (no passed-through output), k = 0, one column, many columns; rows
of one call equal to the same rows called alone, with the x rows staged in
LDS and read from global memory (the summation order does not depend on the
row count or on where x comes from); a reused workspace on two calls in a row,
the second smaller, whose counter is back at zero after each; repeated
calls give the same bits; seeded random shapes; HIP-graph replays; two
calls overlapping on two streams with their own workspaces.
"""
from __future__ import annotations

import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from synth import cases as sc  # noqa: E402


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests import gemv_parity
    from tests import gpu_harness as gh
    return gh, gemv_parity


def counters_left(workspace) -> int:
    """Non-zero bytes in a workspace's arrival-counter header (its size is
    what a [n][k] workspace needs for one normed value, less that value);
    every call must leave the norm's and the tiles' counters at zero."""
    import qk_rope_paged_amd as qrp
    hdr = qrp.gemv_norm_workspace_bytes(1, 1) - 4
    return int(torch.count_nonzero(workspace[:hdr]).item())


def run_and_compare(case, workspace=None, no_workspace=False):
    gh, gp = _gpu()
    print(f"[gemv] {case.name} dtype={case.dtype} m={case.m} k={case.k} n={case.n} "
          f"n_normed={case.n_normed}", flush=True)
    res = oracle.run_gemv(case)
    assert res.status == 0
    dg = gh.upload_gemv(case, workspace=workspace)
    gh.run_gemv(dg, no_workspace=no_workspace)
    torch.cuda.synchronize()
    rep = gp.check(case, res, gh.to_numpy_bits(dg.normed, case.dtype),
                   gh.to_numpy_bits(dg.unnormed, case.dtype))
    left = counters_left(dg.workspace)
    assert left == 0, f"{left} arrival counter bytes left non-zero"
    print(f"[gemv] {case.name} ok {rep}", flush=True)
    return dg, rep


@pytest.mark.parametrize("small", [True, False])
def test_bench_shape(small):
    run_and_compare(sc.gemv_norm(small=small))


@pytest.mark.parametrize("dtype", [sc.F32, sc.BF16, sc.F16])
@pytest.mark.parametrize("m", [1, 2, 3, 5, 8])
def test_rows_dtypes_and_ragged_sizes(dtype, m):
    E = 4 if dtype == sc.F32 else 8
    k = E * (64 * 3 + 5)                 # three full chunk rounds and a ragged one
    case = sc.make_gemv_case(f"rows_{dtype}_{m}", 20 + m, dtype, m=m, k=k, n=333, n_normed=201,
                             epsilon=1e-5, x_pad=E, w_pad=2 * E, out_pad=3)
    run_and_compare(case)


def test_nothing_normed_needs_no_workspace():
    run_and_compare(sc.make_gemv_case("no_norm", 31, sc.BF16, m=2, k=512, n=300, n_normed=0),
                    no_workspace=True)


@pytest.mark.parametrize("m", [1, 4])
def test_everything_normed(m):
    run_and_compare(sc.make_gemv_case("all_norm", 32, sc.BF16, m=m, k=1024, n=777, n_normed=777))


def test_k_zero_gives_zeros():
    # padded strides keep the operand buffers non-empty (a real device address)
    case = sc.make_gemv_case("k0", 33, sc.F32, m=2, k=0, n=10, n_normed=4, epsilon=1e-3,
                             x_pad=4, w_pad=4)
    dg, _ = run_and_compare(case)
    gh, _ = _gpu()
    assert np.all(gh.to_numpy_bits(dg.normed, sc.F32)[:, :4] == 0)
    assert np.all(gh.to_numpy_bits(dg.unnormed, sc.F32)[:, :6] == 0)


def test_one_column_and_many_columns():
    run_and_compare(sc.make_gemv_case("n1", 34, sc.BF16, m=1, k=256, n=1, n_normed=1))
    run_and_compare(sc.make_gemv_case("n1u", 35, sc.BF16, m=3, k=256, n=1, n_normed=0),
                    no_workspace=True)
    run_and_compare(sc.make_gemv_case("wide", 36, sc.BF16, m=1, k=128, n=40000,
                                      n_normed=30001))


@pytest.mark.parametrize("k", [2048, 7168])     # x rows through LDS (32 KB) / global memory
def test_rows_match_single_row_calls(k):
    gh, _ = _gpu()
    case = sc.make_gemv_case("rows8", 37, sc.BF16, m=8, k=k, n=500, n_normed=300)
    dg = gh.upload_gemv(case)
    gh.run_gemv(dg)
    for i in (0, 3, 7):
        one = sc.make_gemv_case("rows8", 37, sc.BF16, m=8, k=k, n=500, n_normed=300)
        one.m, one.x = 1, case.x[i:i + 1]
        d1 = gh.upload_gemv(one)
        gh.run_gemv(d1)
        torch.cuda.synchronize()
        assert torch.equal(d1.normed[0], dg.normed[i]), i
        assert torch.equal(d1.unnormed[0], dg.unnormed[i]), i


@pytest.mark.parametrize("m,k", [(4, 7168), (8, 7168), (3, 16384), (2, 64), (4, 8192), (4, 8000)])
def test_x_rows_staged_in_lds_or_read_from_global_memory(m, k):
    # the x rows go through LDS up to 63 KB (4 x 14 KB, 2 x 128 B, 4 x 15.6 KB)
    # and through global memory past it (8 x 14 KB, 3 x 32 KB, 4 x 16 KB)
    run_and_compare(sc.make_gemv_case(f"x_{m}_{k}", 41 + m, sc.BF16, m=m, k=k, n=300,
                                      n_normed=200))


@pytest.mark.parametrize("kc", [1, 64, 65, 1024, 1025, 1500])
def test_chunk_rounds_of_a_wave(kc):
    # a one-row wave loads 16 chunks per lane per round (1024 chunks): a
    # partial first round, exactly one and two rounds, and ragged ones
    for dtype in (sc.F32, sc.BF16):
        E = 4 if dtype == sc.F32 else 8
        run_and_compare(sc.make_gemv_case(f"rounds_{dtype}_{kc}", 50 + kc % 7, dtype, m=1,
                                          k=E * kc, n=150, n_normed=90))


@pytest.mark.parametrize("m,n,n_normed", [(1, 5000, 10), (3, 5000, 3), (1, 600, 599),
                                           (2, 3000, 2999), (8, 70, 1)])
def test_few_normed_columns_among_many(m, n, n_normed):
    # fewer blocks hold normed columns than the grid has (the arrivals),
    # and the passed-through columns take several rounds of the grid
    run_and_compare(sc.make_gemv_case(f"few_{m}_{n}_{n_normed}", 60 + m, sc.BF16, m=m, k=512,
                                      n=n, n_normed=n_normed))


def test_workspace_reused_on_two_calls_the_second_smaller():
    gh, _ = _gpu()
    big = sc.make_gemv_case("ws_big", 38, sc.BF16, m=4, k=1024, n=900, n_normed=700)
    small = sc.make_gemv_case("ws_small", 39, sc.BF16, m=2, k=512, n=200, n_normed=130)
    dg, _ = run_and_compare(big)
    run_and_compare(small, workspace=dg.workspace)


def test_repeated_calls_give_the_same_bits():
    gh, _ = _gpu()
    case = sc.gemv_norm(small=True)
    dg = gh.upload_gemv(case)
    gh.run_gemv(dg)
    torch.cuda.synchronize()
    first = (dg.normed.clone(), dg.unnormed.clone())
    for _ in range(5):
        gh.run_gemv(dg)
    torch.cuda.synchronize()
    assert torch.equal(first[0], dg.normed) and torch.equal(first[1], dg.unnormed)


def _random_case(i: int):
    rng = np.random.default_rng([4099, i])
    dtype = (sc.F32, sc.BF16, sc.F16)[int(rng.integers(3))]
    E = 4 if dtype == sc.F32 else 8
    m = int(rng.integers(1, 9))
    k = E * int(rng.integers(0, 400))
    n = int(rng.integers(1, 3000))
    nn = int(rng.choice([0, n, int(rng.integers(0, n + 1))]))
    return sc.make_gemv_case(f"rand_gemv_{i}", 600 + i, dtype, m=m, k=k, n=n, n_normed=nn,
                             epsilon=float(rng.choice([1e-6, 1e-3])),
                             weight_offset=float(rng.choice([0.0, 0.5])),
                             x_pad=E * int(rng.integers(0, 3)) + (E if k == 0 else 0),
                             w_pad=E * int(rng.integers(0, 3)) + (E if k == 0 else 0),
                             out_pad=int(rng.integers(0, 3)))


# QRP_RANDOM_CASES sets the count (1000: a soak of the arrival counter and the bar)
@pytest.mark.parametrize("i", range(int(os.environ.get("QRP_RANDOM_CASES", "24"))))
def test_random_shapes(i):
    case = _random_case(i)
    run_and_compare(case, no_workspace=case.n_normed == 0)


def test_graph_replays_match_eager():
    # a captured launch reuses its workspace on every replay: the counter
    # must be back at zero each time
    gh, _ = _gpu()
    case = sc.gemv_norm(small=True)
    eager = gh.upload_gemv(case)
    gh.run_gemv(eager)
    torch.cuda.synchronize()
    dg = gh.upload_gemv(case)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        gh.run_gemv(dg, stream=s)
    for _ in range(3):
        dg.normed.fill_(0)
        dg.unnormed.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dg.normed, eager.normed) and torch.equal(dg.unnormed, eager.unnormed)
        assert counters_left(dg.workspace) == 0


def test_overlapping_calls_on_two_streams_with_their_own_workspaces():
    # no state is shared between calls but the workspace: two calls in
    # flight together, each with its own, give the results of one at a time
    gh, _ = _gpu()
    cases = [sc.gemv_norm(small=True), sc.make_gemv_case("other", 40, sc.BF16, m=3, k=1536,
                                                         n=1000, n_normed=640)]
    ref = []
    for c in cases:
        d = gh.upload_gemv(c)
        gh.run_gemv(d)
        torch.cuda.synchronize()
        ref.append(d)
    devs = [gh.upload_gemv(c) for c in cases]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for _ in range(20):
        for d, s in zip(devs, streams):
            gh.run_gemv(d, stream=s)
    torch.cuda.synchronize()
    for d, r in zip(devs, ref):
        assert torch.equal(d.normed, r.normed) and torch.equal(d.unnormed, r.unnormed)
        assert counters_left(d.workspace) == 0


@pytest.mark.parametrize("dtype,x_scale,w_std", [(sc.F16, 100.0, 1e-5), (sc.BF16, 1e30, 1e-39)])
def test_subnormal_weights_are_not_flushed(dtype, x_scale, w_std):
    # every weight is subnormal in the dtype; x is large, so the products are
    # ordinary numbers: a flush of subnormal inputs would lose all of them
    from synth import prng
    case = sc.make_gemv_case(f"subnormal_{dtype}", 50, dtype, m=2, k=512, n=96, n_normed=40)
    k, n = case.k, case.n
    case.x = sc.to_bits(prng.normal(50, 9, 2 * k).reshape(2, k) * x_scale, dtype)
    w = prng.normal(50, 10, n * k, std=w_std).reshape(n, k)
    case.w = sc.to_bits(w, dtype)
    vals = sc.bits_to_f64(case.w, dtype)
    tiny = 2.0 ** -14 if dtype == sc.F16 else 2.0 ** -126
    assert np.all(np.abs(vals) < tiny) and np.count_nonzero(vals) > 0.9 * vals.size
    run_and_compare(case)


# ---- W stored [k][n] (transpose_b = 0; MatmulFusedPartialRMSNorm page, Parameters) ----

@pytest.mark.parametrize("small", [True, False])
def test_w_stored_k_by_n_bench_shape(small):
    run_and_compare(sc.gemv_norm(small=small, transpose_b=False))


@pytest.mark.parametrize("dtype", [sc.F32, sc.BF16, sc.F16])
@pytest.mark.parametrize("m", [1, 2, 3, 5, 8])
def test_w_stored_k_by_n_rows_dtypes_and_ragged_sizes(dtype, m):
    # k over several slices, each a whole round of the block's 512 rows and
    # a ragged one; n not a multiple of the tile, W rows padded
    E = 4 if dtype == sc.F32 else 8
    k = E * (256 * 2 + 5)
    case = sc.make_gemv_case(f"t_rows_{dtype}_{m}", 70 + m, dtype, m=m, k=k, n=333, n_normed=201,
                             epsilon=1e-5, x_pad=E, w_pad=3 * E - 333 % E, out_pad=3,
                             transpose_b=False)
    run_and_compare(case)


@pytest.mark.parametrize("n,w_pad", [(150, 2), (16, 0), (1, 7), (8, 0), (17, 7)])
def test_w_stored_k_by_n_last_unit_at_the_row_end(n, w_pad):
    # the last tile's chunks from the row stride on are not read (n = 150,
    # stride 152: the tile's fourth chunk onward; n = 1, stride 8: all but
    # the first)
    case = sc.make_gemv_case(f"t_end_{n}", 80 + n, sc.BF16, m=1, k=512, n=n,
                             n_normed=min(n, 5), w_pad=w_pad, transpose_b=False)
    assert case.w.shape[1] % 8 == 0
    run_and_compare(case)


@pytest.mark.parametrize("m,nn", [(2, 300), (8, 300), (8, 1100)])
def test_w_stored_k_by_n_rows_match_single_row_calls(m, nn):
    # k in two slices; with 8 rows of 1100 normed columns the slices' sums
    # meet per tile first, with one row they meet at the norm's counter
    # directly: the sums are added in the same order either way
    gh, _ = _gpu()
    mk = lambda: sc.make_gemv_case("t_rows", 90, sc.BF16, m=m, k=2048, n=1200, n_normed=nn,
                                   w_pad=0, transpose_b=False)
    case = mk()
    dg = gh.upload_gemv(case)
    gh.run_gemv(dg)
    for i in range(m):
        one = mk()
        one.m, one.x = 1, case.x[i:i + 1]
        d1 = gh.upload_gemv(one)
        gh.run_gemv(d1)
        torch.cuda.synchronize()
        assert torch.equal(d1.normed[0], dg.normed[i]), i
        assert torch.equal(d1.unnormed[0], dg.unnormed[i]), i


def test_w_stored_k_by_n_nothing_normed_and_k_zero():
    # nothing normed: the slices' sums still meet in the workspace
    run_and_compare(sc.make_gemv_case("t_nonorm", 91, sc.BF16, m=2, k=4096, n=300, n_normed=0,
                                      w_pad=4, transpose_b=False))
    case = sc.make_gemv_case("t_k0", 92, sc.F32, m=2, k=0, n=10, n_normed=4, epsilon=1e-3,
                             x_pad=4, w_pad=2, transpose_b=False)
    # k = 0: W has no rows; keep the buffer non-empty (a real device address)
    case.w = np.full((1, 12), sc.SENTINEL[sc.F32], dtype=case.w.dtype)
    dg, _ = run_and_compare(case)
    gh, _ = _gpu()
    assert np.all(gh.to_numpy_bits(dg.normed, sc.F32)[:, :4] == 0)


# QRP_RANDOM_CASES sets twice the count here
@pytest.mark.parametrize("i", range(int(os.environ.get("QRP_RANDOM_CASES", "24")) // 2))
def test_w_stored_k_by_n_random_shapes(i):
    rng = np.random.default_rng([4111, i])
    dtype = (sc.F32, sc.BF16, sc.F16)[int(rng.integers(3))]
    E = 4 if dtype == sc.F32 else 8
    m = int(rng.integers(1, 9))
    k = E * int(rng.integers(1, 700))
    n = int(rng.integers(1, 3000))
    nn = int(rng.choice([0, n, int(rng.integers(0, n + 1))]))
    case = sc.make_gemv_case(f"t_rand_{i}", 700 + i, dtype, m=m, k=k, n=n, n_normed=nn,
                             epsilon=float(rng.choice([1e-6, 1e-3])),
                             x_pad=E * int(rng.integers(0, 3)),
                             w_pad=(-n) % E + E * int(rng.integers(0, 3)),
                             out_pad=int(rng.integers(0, 3)), transpose_b=False)
    run_and_compare(case)


@pytest.mark.parametrize("dtype,m,k,n,nn", [
    (sc.BF16, 1, 16384, 64, 64),     # one tile: 16 slices
    (sc.F16, 3, 24576, 130, 100),    # three tiles, the last of 2 columns: many slices
    (sc.F32, 2, 8192, 40, 33),       # fp32 tiles of 32 columns
    (sc.BF16, 2, 512 * 7 + 8, 2112, 1536),   # the last slice 8 rows longer than a round
    (sc.BF16, 8, 4096, 2112, 1536),  # 8 rows of y past the LDS copy: tiles meet first
    (sc.F16, 4, 8192, 1000, 700),    # many slice sums: tiles meet first
    (sc.BF16, 1, 8, 700, 500),       # one row group's rows: one slice
    (sc.BF16, 2, 1024, 64 * 260, 64 * 200),  # more tiles than compute units: one slice
    (sc.F32, 1, 4, 33, 33),          # k of one chunk
])
def test_w_stored_k_by_n_slices(dtype, m, k, n, nn):
    # how k is cut into slices follows from n, k and the dtype; each case
    # holds a different count, down to one, and the counters end at zero
    E = 4 if dtype == sc.F32 else 8
    run_and_compare(sc.make_gemv_case(f"t_slices_{dtype}_{k}_{n}", 95, dtype, m=m, k=k, n=n,
                                      n_normed=nn, w_pad=(-n) % E, transpose_b=False))

"""GPU parity of the padded continuous-batching op
(generic_fused_qk_rope_bshd_continuous_batch page) against the CPU oracle,
plus GPU-vs-GPU relations.

Cases: the workload at reduced and full size, every dtype and head_dim in
both layouts with tables of the op's dtype and of binary32, partial rope,
valid lengths of 0 and past the padded length, a one-row grid (decode),
out-of-range metadata, and the equivalence with the ragged in-place op when
every row is real.
"""
from __future__ import annotations

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


def run_and_compare(case):
    gh, parity = _gpu()
    print(f"[bshd] {case.name} dtype={case.dtype} B={case.batch} S={case.seq_len} "
          f"seed={case.seed}", flush=True)
    res = oracle.run_case(case)
    dc = gh.upload(case)
    gh.run(dc)
    torch.cuda.synchronize()
    rep = parity.compare(case, dc, res)
    print(f"[bshd] {case.name} ok {dict(rep)}", flush=True)
    return rep


def _case(name, seed, dtype, valid, S, clen, D=128, R=None, il=True, Hq=6, Hk=2, capacity=512,
          L=2, layer=1, msl=512, freq_dtype=None):
    return sc.make_bshd_case(name, seed, dtype, list(valid), S, list(clen), Hq=Hq, Hk=Hk, D=D,
                             rope_dim=R or D, interleaved=il, theta=1e4, max_seq_len=msl,
                             capacity=capacity, L=L, layer=layer, freq_dtype=freq_dtype)


@pytest.mark.parametrize("seed", [None, 106])
def test_bshd_small_workload(seed):
    run_and_compare(sc.bshd(small=True) if seed is None else sc.bshd(seed, small=True))


def test_bshd_full_size_workload():
    rep = run_and_compare(sc.bshd())
    assert rep["q_passed_rows"] > 0


@pytest.mark.parametrize("dtype", [sc.F32, sc.BF16, sc.F16])
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("il", [True, False])
def test_bshd_dtypes_head_dims_and_layouts(dtype, D, il):
    run_and_compare(_case(f"bshd_{dtype}_{D}_{il}", 40, dtype, [5, 0, 17, 30, 2], 24,
                          [0, 9, 100, 3, 480], D=D, il=il))


@pytest.mark.parametrize("dtype", [sc.F32, sc.BF16, sc.F16])
@pytest.mark.parametrize("il", [True, False])
def test_bshd_binary32_table_and_partial_rope(dtype, il):
    R = 16 if dtype == sc.F32 else 32
    run_and_compare(_case(f"bshd_partial_{dtype}_{il}", 41, dtype, [11, 3, 40], 19, [4, 0, 77],
                          R=R, il=il, freq_dtype=sc.F32))


def test_bshd_valid_lengths_zero_and_past_the_padded_length():
    run_and_compare(_case("bshd_edges", 42, sc.BF16, [0, 64, 7, 0, 200], 9, [3, 1, 0, 8, 300]))


def test_bshd_all_rows_padded():
    run_and_compare(_case("bshd_none", 43, sc.BF16, [0, 0, 0], 16, [5, 0, 2]))


def test_bshd_one_row_grid_decode():
    B = 64
    valid = prng.integers(44, 1, B, 0, 1)
    clen = prng.integers(44, 2, B, 0, 8000)
    run_and_compare(_case("bshd_decode", 44, sc.BF16, valid, 1, clen, Hq=32, Hk=8, capacity=8192,
                          L=1, layer=0, msl=8192))


def test_bshd_out_of_range_rows_are_skipped():
    gh, parity = _gpu()
    good = _case("bshd_oob", 45, sc.BF16, [6, 4, 5], 8, [10, 30, 2])
    res = oracle.run_case(good)
    # sequence 1 now starts at position 509: its real rows 3.. fall past max_seq_len 512
    bad = _case("bshd_oob", 45, sc.BF16, [6, 4, 5], 8, [10, 30, 2])
    bad.caches[0].cache_lengths = np.array([10, 509, 2], np.uint32)
    dc = gh.upload(bad)
    gh.run(dc)
    torch.cuda.synchronize()
    S, D, Hq = 8, 128, 6
    q = gh.to_numpy_bits(dc.q_out_rows(0), sc.BF16)
    sent = sc.SENTINEL[sc.BF16]
    # out-of-range real rows write nothing; padded rows of sequence 1 are still copied
    assert np.all(q[S + 3:S + 4] == sent)
    assert np.array_equal(q[S + 4:2 * S], bad.buf[S + 4:2 * S])
    # sequences 0 and 2 match the oracle run on the good metadata
    others = [t for t in range(3 * S) if not S <= t < 2 * S]
    tr = res.traces[0]
    ok = parity.tol_ok(q[others].reshape(-1, D), tr["q_exact"][others].reshape(-1, D),
                       tr["q_mag"][others].reshape(-1, D), sc.BF16, 1)
    assert ok.all()


def test_bshd_equals_ragged_in_place_op_when_every_row_is_real():
    """With every valid length = S the padded grid is a ragged batch with
    offsets b*S: the ragged norm op with no gammas, K in the cache and Q
    from the same rows must give the same bits."""
    gh, _ = _gpu()
    import qk_rope_paged_amd as qrp
    B, S = 5, 37
    case = _case("bshd_eq", 46, sc.BF16, [S] * B, S, [0, 12, 99, 3, 250], Hq=8, Hk=2, il=False)
    a, b = gh.upload(case), gh.upload(case)
    gh.run(a)
    D = 128
    band = qrp.Band(q_col=0, n_q_heads=8, k_col=-1, v_col=-1, q_gamma=None, k_gamma=None,
                    epsilon=1e-6, cache=b.caches[0].desc, q_output=b.q_out_rows(0),
                    q_out_row_stride=8 * D)
    qrp.qk_rmsnorm_rope_paged(b.buf, qrp.QRP_BF16, B * S, 8 * D, band, 0.0, True, b.offsets, B,
                              gh.rope_of(b), case.layer_idx)
    torch.cuda.synchronize()
    for x, y in zip([a.q_out[0], a.caches[0].pool], [b.q_out[0], b.caches[0].pool]):
        assert torch.equal(x, y)

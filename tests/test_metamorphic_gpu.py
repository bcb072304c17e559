"""GPU-vs-GPU relations that must hold bit for bit, plus launch-path checks.

* the dual band equals its main-band call followed by its index-band call
  (fused_dual_qk_rms_norm_rope_ragged_paged page, Summary: one launch in
  place of two);
* the norm op with no gammas and K/V from the buffer equals the rope-only op;
* half-split RoPE equals interleaved RoPE on each head's halves interleaved;
* every launch configuration (passes per wave, waves per block,
  XCD-contiguous remap) gives the same bits;
* the device validator accepts good metadata and rejects a shared row;
* tokens whose metadata is out of range are skipped: nothing is written for
  them and every other token is exact;
* a call on a non-default stream, and a HIP graph of the in-place radd
  replayed with eager work between replays, match eager execution.
"""
from __future__ import annotations

import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from synth import cases as sc  # noqa: E402


def _env():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import qk_rope_paged_amd as qrp
    from tests import gpu_harness as gh
    from tests import parity
    return qrp, gh, parity


def _bits(t, dtype):
    from tests import gpu_harness as gh
    return gh.to_numpy_bits(t, dtype)


def _snapshot(dc):
    out = [_bits(q, dc.case.dtype) for q in dc.q_out]
    out += [_bits(c.pool, dc.case.dtype) for c in dc.caches]
    return out


def _assert_same(a, b, what):
    assert len(a) == len(b)
    for i, (x, y) in enumerate(zip(a, b)):
        assert np.array_equal(x, y), f"{what}: buffer {i} differs"


def test_dual_band_equals_main_then_index_call():
    qrp, gh, _ = _env()
    case = sc.dual(small=True)
    fused, split = gh.upload(case), gh.upload(case)
    gh.run(fused)
    dt = gh.QRP_DT[case.dtype]
    for i in (0, 1):
        qrp.qk_rmsnorm_rope_paged(split.buf, dt, case.T, case.row_stride, gh.band_of(split, i),
                                  case.weight_offset, case.multiply_before_cast, split.offsets,
                                  case.batch, gh.rope_of(split), case.layer_idx)
    torch.cuda.synchronize()
    _assert_same(_snapshot(fused), _snapshot(split), "dual vs two single-band calls")


def test_norm_op_without_gammas_equals_rope_split_store():
    qrp, gh, _ = _env()
    case = sc.prefill(small=True)
    a, b = gh.upload(case), gh.upload(case)
    gh.run(a)
    D, Hq, Hk = 128, case.n_q_heads, case.caches[0].num_kv_heads
    band = qrp.Band(q_col=0, n_q_heads=Hq, k_col=Hq * D, v_col=(Hq + Hk) * D, q_gamma=None,
                    k_gamma=None, epsilon=1e-6, cache=b.caches[0].desc, q_output=b.q_out_rows(0),
                    q_out_row_stride=case.q_out_row_stride)
    qrp.qk_rmsnorm_rope_paged(b.buf, gh.QRP_DT[case.dtype], case.T, case.row_stride, band, 0.0,
                              True, b.offsets, case.batch, gh.rope_of(b), case.layer_idx)
    torch.cuda.synchronize()
    _assert_same(_snapshot(a), _snapshot(b), "norm without gammas vs rope_split_store")


@pytest.mark.parametrize("R", [128, 64])
def test_half_split_equals_permuted_interleaved(R):
    _, gh, _ = _env()
    mk = lambda il: sc.make_store_case("perm", 31, sc.BF16, [40, 7, 0, 19], [0, 100, 3, 250],
                                       Hq=8, Hk=2, D=128, rope_dim=R, interleaved=il, theta=5e5,
                                       max_seq_len=512, P=32, L=1, layer=0)
    hs, il = mk(False), mk(True)
    D, H = 128, 8 + 2 * 2
    perm = np.arange(D)
    perm[0:R:2] = np.arange(R // 2)
    perm[1:R:2] = np.arange(R // 2) + R // 2
    il.buf = np.ascontiguousarray(hs.buf.reshape(hs.T, H, D)[:, :, perm].reshape(hs.T, H * D))
    dh, di = gh.upload(hs), gh.upload(il)
    gh.run(dh)
    gh.run(di)
    torch.cuda.synchronize()
    inv = np.argsort(perm)
    q_h = _bits(dh.q_out_rows(0), sc.BF16).reshape(hs.T, 8, D)
    q_i = _bits(di.q_out_rows(0), sc.BF16).reshape(hs.T, 8, D)[:, :, inv]
    assert np.array_equal(q_h, q_i)
    shape = hs.caches[0].shape
    k_h = _bits(dh.caches[0].pool, sc.BF16).reshape(shape)[:, 0]
    k_i = _bits(di.caches[0].pool, sc.BF16).reshape(shape)[:, 0][..., inv]
    assert np.array_equal(k_h, k_i)


@pytest.mark.parametrize("workload", ["prefill", "decode", "dual", "radd", "bshd", "prefill_tp8", "dual_tp8"])
def test_launch_configuration_does_not_change_bits(workload, monkeypatch):
    _, gh, _ = _env()
    case = sc.WORKLOADS[workload](small=True)
    ref = None
    for remap in ("0", "1", "2"):
        for ppw in ("0", "1", "2", "3"):
            for wpb in ("0", "1", "2", "4"):
                dc = gh.upload(case)
                with gh.knobs(remap, ppw, wpb):
                    gh.run(dc)
                torch.cuda.synchronize()
                snap = _snapshot(dc)
                if ref is None:
                    ref = snap
                else:
                    _assert_same(ref, snap, f"{workload} remap={remap} ppw={ppw} wpb={wpb}")


@pytest.mark.parametrize("workload", ["prefill", "dual", "bshd", "prefill_tp8", "dual_tp8",
                                      "prefill_fp8"])
def test_one_pass_tail_does_not_change_bits(workload):
    """The last units of a multi-pass launch may run one pass per wave
    (QRP_KNOB_TAIL_UNITS): every tail size, from none to the whole launch,
    with every pass count and XCD mapping, gives the same bits."""
    _, gh, _ = _env()
    case = sc.WORKLOADS[workload](small=True)
    ref = None
    for remap in ("0", "1"):
        for ppw in ("0", "2", "3"):
            for tail in (0, 1, 2, 5, 33, 10 ** 6):
                dc = gh.upload(case)
                with gh.knobs(remap, ppw, tail=tail):
                    gh.run(dc)
                torch.cuda.synchronize()
                snap = _snapshot(dc)
                if ref is None:
                    ref = snap
                else:
                    _assert_same(ref, snap, f"{workload} remap={remap} ppw={ppw} tail={tail}")


@pytest.mark.parametrize("workload", ["prefill", "decode", "dual", "radd", "bshd", "radd_fp8",
                                      "dual_tp8"])
def test_reserved_lds_does_not_change_bits(workload):
    """LDS reserved per block (QRP_KNOB_LDS_BYTES; radd over a plain cache
    reserves 32 KB by default) caps the resident blocks and changes nothing
    else: every size gives the same bits."""
    _, gh, _ = _env()
    case = sc.WORKLOADS[workload](small=True)
    ref = None
    for lds in (-1, 0, 1, 16384, 32768, 49152):
        for wpb in ("0", "1"):
            dc = gh.upload(case)
            with gh.knobs(wpb=wpb, lds=lds):
                gh.run(dc)
            torch.cuda.synchronize()
            snap = _snapshot(dc)
            if ref is None:
                ref = snap
            else:
                _assert_same(ref, snap, f"{workload} lds={lds} wpb={wpb}")


def test_validate_on_device():
    qrp, gh, _ = _env()
    case = sc.prefill(small=True)
    dc = gh.upload(case)
    c = dc.caches[0]
    assert qrp.qrp_validate(dc.offsets, case.batch, case.T, 0, c.desc, case.max_seq_len) == 0
    # make sequence 1 write the page sequence 0 starts in, at the same rows
    tab = c.lookup_table.clone()
    tab[1, 0] = tab[0, 0]
    bad = qrp.PagedCache(**{**c.desc.__dict__, "lookup_table": tab})
    assert qrp.qrp_validate(dc.offsets, case.batch, case.T, 0, bad, case.max_seq_len) == \
        qrp.QRP_EDATA
    assert "same cache row" in qrp.last_error()


@pytest.mark.parametrize("pack", ["0", "1"])
def test_out_of_range_tokens_are_skipped(pack, monkeypatch):
    """Per-token layout: the token's wave leaves; token-packed layout: the
    token's rows stay in their wave, masked (QRP_PACK forces either)."""
    _, gh, parity = _env()
    monkeypatch.setattr(gh, "OVERRIDES", {"pack": int(pack)})
    lens, clen = [6, 9, 4], [10, 30, 5]
    good = sc.make_store_case("oob", 41, sc.BF16, lens, clen, Hq=8, Hk=2, D=128, rope_dim=128,
                              interleaved=True, theta=1e4, max_seq_len=512, P=16, L=1, layer=0)
    res = oracle.run_case(good)
    # sequence 1 now starts at position 510: its tokens 2.. fall past max_seq_len
    bad = sc.make_store_case("oob", 41, sc.BF16, lens, clen, Hq=8, Hk=2, D=128, rope_dim=128,
                             interleaved=True, theta=1e4, max_seq_len=512, P=16, L=1, layer=0)
    bad.caches[0].cache_lengths = np.array([10, 510, 5], np.uint32)
    dc = gh.upload(bad)
    gh.run(dc)
    torch.cuda.synchronize()
    D = 128
    q = _bits(dc.q_out_rows(0), sc.BF16)
    pool = _bits(dc.caches[0].pool, sc.BF16)
    sent = sc.SENTINEL[sc.BF16]
    t1 = range(6, 15)                    # tokens of sequence 1
    # tokens at positions >= 512 wrote nothing
    for t in t1:
        if 510 + (t - 6) >= 512:
            assert np.all(q[t] == sent)
    # every token of sequences 0 and 2 matches the oracle exactly as in the valid batch
    others = [t for t in range(good.T) if t not in t1]
    tr = res.traces[0]
    ok = parity.tol_ok(q[others, :8 * D].reshape(-1, D), tr["q_exact"][others].reshape(-1, D),
                       tr["q_mag"][others].reshape(-1, D), sc.BF16, 1)
    assert ok.all()
    for t in others:
        for h in range(2):
            v = tr["v_row_off"][t, h]
            assert np.array_equal(pool[v:v + D], res.pools[0].reshape(-1)[v:v + D])


def test_non_default_stream():
    _, gh, parity = _env()
    case = sc.prefill(small=True)
    res = oracle.run_case(case)
    dc = gh.upload(case)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        gh.run(dc, stream=s)
    s.synchronize()
    parity.compare(case, dc, res)


def test_graph_replays_of_radd_match_eager():
    _, gh, _ = _env()
    case = sc.radd(small=True)
    eager, graphed = gh.upload(case), gh.upload(case)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        gh.run(graphed, stream=s)
    torch.cuda.synchronize()
    for i in range(3):
        g.replay()
        torch.cuda.synchronize()
        gh.run(eager)
        scratch = torch.ones(1 << 20, device="cuda").mul_(2.0)   # unrelated eager work
        torch.cuda.synchronize()
        del scratch
        a = _bits(eager.caches[0].pool, case.dtype)
        b = _bits(graphed.caches[0].pool, case.dtype)
        assert np.array_equal(a, b), f"replay {i} differs from eager"


@pytest.mark.parametrize("il", [True, False])
def test_trailing_rope_equals_leading_rope_on_rolled_heads(il):
    """Rolling every head by head_dim - rope_dim maps the trailing-dims
    convention onto the leading one: two GPU runs agree bit for bit."""
    _, gh, _ = _env()
    D, R, Hq, Hk = 128, 64, 8, 2
    mk = lambda tail: sc.make_store_case("roll", 33, sc.BF16, [40, 7, 0, 19], [0, 100, 3, 250],
                                         Hq=Hq, Hk=Hk, D=D, rope_dim=R, interleaved=il, theta=5e5,
                                         max_seq_len=512, P=32, L=1, layer=0, rope_tail=tail)
    tail, lead = mk(True), mk(False)
    H = Hq + 2 * Hk
    lead.buf = np.ascontiguousarray(
        np.roll(tail.buf.reshape(tail.T, H, D), -(D - R), axis=2).reshape(tail.T, H * D))
    dt, dl = gh.upload(tail), gh.upload(lead)
    gh.run(dt)
    gh.run(dl)
    torch.cuda.synchronize()
    qt = _bits(dt.q_out_rows(0), sc.BF16).reshape(tail.T, Hq, D)
    ql = np.roll(_bits(dl.q_out_rows(0), sc.BF16).reshape(lead.T, Hq, D), D - R, axis=2)
    assert np.array_equal(qt, ql)
    shape = tail.caches[0].shape
    kt = _bits(dt.caches[0].pool, sc.BF16).reshape(shape)[:, 0]
    kl = np.roll(_bits(dl.caches[0].pool, sc.BF16).reshape(shape)[:, 0], D - R, axis=-1)
    assert np.array_equal(kt, kl)


@pytest.mark.parametrize("workload", ["prefill", "decode", "dual", "radd", "bshd", "prefill_tp8",
                                      "decode_tp8", "dual_tp8", "prefill_fp8", "decode_fp8",
                                      "dual_fp8", "radd_fp8", "bshd_fp8"])
def test_token_packed_layout_gives_the_same_bits(workload, monkeypatch):
    """The token-packed layout (a pass is one head of a block of consecutive
    tokens) and the per-token layout compute every row alike: forced on and
    off, every output row, cache element and scale is bit-identical, also for
    head counts that would not pick packing by themselves."""
    _, gh, _ = _env()
    case = sc.WORKLOADS[workload](small=True)
    snaps = []
    for pack in ("0", "1"):
        dc = gh.upload(case)
        with gh.knobs(pack=pack):
            gh.run(dc)
        torch.cuda.synchronize()
        snap = [gh.to_numpy_bits(q, case.q_dtype) for q in dc.q_out]
        snap += [gh.to_numpy_bits(c.pool, c.host.dtype) for c in dc.caches]
        snap += [gh.to_numpy_bits(c.scales, c.host.scale_dtype) for c in dc.caches
                 if c.scales is not None]
        snaps.append(snap)
    _assert_same(snaps[0], snaps[1], f"{workload}: packed and per-token layouts")

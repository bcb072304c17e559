"""Seeded random combinations of every option, GPU against the CPU oracle.

The other GPU tests vary one or two options around a workload; this one
draws, per case, the op and every option it takes at once: input dtype,
head_dim, rope width and placement (leading or trailing dims), layout,
freqs-table dtype, cache dtype (plain or FP8 with f32 / bf16 scales, the
dual band's two caches sometimes one of each), Q
output dtype, page size (1, powers of two and others), head counts, batch
size on both sides of the small-batch threshold and up to 512 sequences,
ragged and empty sequences,
cache lengths up to the table's end, and the norm op's switches; odd cases
force the per-token layout, even ones let the library pick (mostly the
token-packed layout at these head counts), and every third case also draws
the launch shape (passes per wave, the one-pass tail's size, waves per
block, the XCD mapping, LDS reserved per block), which never changes the
bits.  Every case
is valid by construction (positions stay below max_seq_len, rope widths are
multiples of two 16-byte chunks); each is compared element by element with
the parity bar of tests/parity.py (which widens it for normalised values
next to a midpoint of multiply_before_cast = false's first rounding, as that
module derives).  The draws come from numpy generators
keyed by the case index, so a failure names a reproducible case.
"""
from __future__ import annotations

import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from synth import cases as sc  # noqa: E402

OPS = ("store", "norm", "dual", "radd", "bshd")
# cases per op; QRP_RANDOM_CASES=1000 runs the 5,000-case soak
N_PER_OP = int(os.environ.get("QRP_RANDOM_CASES", "24"))
MSL = 512


def _pick(rng, seq):
    return seq[int(rng.integers(len(seq)))]


def _geometry(rng):
    dtype = _pick(rng, (sc.F32, sc.BF16, sc.F16))
    D = _pick(rng, (64, 128, 256))
    ce = 4 if dtype == sc.F32 else 8           # elements per 16-byte chunk
    R = _pick(rng, list(range(2 * ce, D + 1, 2 * ce)))
    return dtype, D, R


def _batch(rng, lo=1, hi=20, max_len=12):
    B = int(rng.integers(lo, hi + 1))            # both sides of the 16-sequence threshold
    top = MSL - max_len
    if rng.random() < 0.2:                       # up to 512 short sequences (deep searches),
        B, max_len, top = int(rng.integers(hi + 1, 513)), 3, 64   # short caches: small pools
    lens = rng.integers(0, max_len + 1, B)
    if lens.sum() == 0:
        lens[int(rng.integers(B))] = 1
    clen = rng.integers(0, top, B)
    clen[rng.random(B) < 0.2] = 0
    return lens, clen


def random_case(op: str, k: int):
    rng = np.random.default_rng([7919, OPS.index(op), k])
    dtype, D, R = _geometry(rng)
    il, tail = bool(rng.integers(2)), bool(rng.integers(2))
    fdt = _pick(rng, (sc.F32, sc.BF16, sc.F16))
    fp8 = bool(rng.integers(2))
    cdt = sc.FP8 if fp8 else None
    sdt = _pick(rng, (sc.F32, sc.BF16))
    P = _pick(rng, (1, 5, 16, 24, 64, 128))
    name = f"rand_{op}_{k}"
    seed = 5000 + 97 * OPS.index(op) + k
    if op == "store":
        lens, clen = _batch(rng)
        q_out = _pick(rng, (None, sc.F32, sc.BF16, sc.F16))
        return sc.make_store_case(name, seed, dtype, lens, clen, Hq=int(rng.integers(1, 10)),
                                  Hk=int(rng.integers(1, 5)), D=D, rope_dim=R, interleaved=il,
                                  theta=1e4, max_seq_len=MSL, P=P, L=2, layer=1, freq_dtype=fdt,
                                  cache_dtype=cdt, scale_dtype=sdt, q_out_dtype=q_out,
                                  rope_tail=tail, row_pad=_pick(rng, (0, 8)))
    if op == "norm":
        lens, clen = _batch(rng)
        return sc.make_norm_case(name, seed, dtype, lens, clen, Hq=int(rng.integers(0, 9)),
                                 Hk=int(rng.integers(1, 5)), D=D, rope_dim=R, interleaved=il,
                                 theta=1e4, max_seq_len=MSL, P=P, L=2, layer=1,
                                 k_in_cache=bool(rng.integers(2)), q_norm=bool(rng.integers(2)),
                                 k_norm=bool(rng.integers(2)), eps=_pick(rng, (1e-6, 1e-3)),
                                 weight_offset=_pick(rng, (0.0, 0.5)),
                                 multiply_before_cast=bool(rng.integers(2)), freq_dtype=fdt,
                                 cache_dtype=cdt, scale_dtype=sdt, rope_tail=tail)
    if op == "dual":
        lens, clen = _batch(rng)
        kw = {}
        if rng.random() < 0.5:                   # the index cache's own lengths
            top = 64 if len(lens) > 20 else MSL - int(lens.max())   # many sequences: small pools
            kw["index_cache_lengths"] = rng.integers(0, top, len(lens))
        idt = cdt
        if rng.random() < 0.3:                   # one plain and one FP8 cache
            idt = None if fp8 else sc.FP8
        return sc.make_dual_case(name, seed, dtype, lens, Hq_main=int(rng.integers(1, 9)),
                                 Hk_main=int(rng.integers(1, 4)), Hq_index=int(rng.integers(1, 5)),
                                 D=D, rope_dim=R, interleaved=il, theta=1e4, max_seq_len=MSL,
                                 P_main=P, P_index=_pick(rng, (1, 8, 24, 64)),
                                 eps_main=1e-6, eps_index=_pick(rng, (1e-6, 1e-3)),
                                 weight_offset=_pick(rng, (0.0, 0.5)),
                                 multiply_before_cast=bool(rng.integers(2)), cache_lengths=clen,
                                 freq_dtype=fdt, main_cache_dtype=cdt, index_cache_dtype=idt,
                                 scale_dtype=sdt, rope_tail=tail, **kw)
    if op == "radd":
        lens, clen_b = _batch(rng)
        off = int(rng.integers(0, 4))
        clen = np.concatenate([rng.integers(0, MSL - 12, off), clen_b,
                               rng.integers(0, MSL - 12, int(rng.integers(0, 3)))])
        return sc.make_radd_case(name, seed, dtype, lens, clen, off, Hk=int(rng.integers(1, 5)),
                                 D=D, P=P, L=2, layer=1, cache_dtype=cdt, scale_dtype=sdt)
    # padded continuous-batching grid
    B = int(rng.integers(1, 12))
    S = int(rng.integers(1, 20))
    valid = rng.integers(0, S + 4, B)              # some past the padded length
    clen = rng.integers(0, MSL - S - 4, B)
    return sc.make_bshd_case(name, seed, dtype, valid, S, clen, Hq=int(rng.integers(1, 9)),
                             Hk=int(rng.integers(1, 4)), D=D, rope_dim=R, interleaved=il,
                             theta=1e4, max_seq_len=MSL, capacity=MSL, L=2, layer=1,
                             freq_dtype=fdt, cache_dtype=cdt, scale_dtype=sdt, rope_tail=tail)


def launch_knobs(op: str, k: int) -> dict:
    """The case's launch-shape overrides (gpu_harness.knobs arguments):
    odd cases force the per-token layout (small head counts would mostly
    pick the token-packed one); every third case draws the rest of the
    shape, with several passes per wave more often than the library would
    pick at these sizes, so that the one-pass tail is exercised."""
    kw = {"pack": 0} if k % 2 else {}
    if k % 3 == 1:
        rng = np.random.default_rng([104729, OPS.index(op), k])
        kw.update(ppw=_pick(rng, ("0", "2", "3")), tail=_pick(rng, (None, 0, 1, 3, 1000)),
                  wpb=_pick(rng, ("0", "1", "2", "4")), remap=_pick(rng, ("0", "1")),
                  lds=_pick(rng, (None, 0, 16384)))
    return kw


@pytest.mark.parametrize("k", range(N_PER_OP))
@pytest.mark.parametrize("op", OPS)
def test_random_combination(op, k, monkeypatch):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests import gpu_harness as gh
    kn = launch_knobs(op, k)
    if kn:
        monkeypatch.setattr(gh, "OVERRIDES", kn)
    from tests import parity
    case = random_case(op, k)
    print(f"[rand] {case.name} dtype={case.dtype} D={case.caches[0].head_dim} "
          f"R={case.rope_dim} il={case.interleaved} tail={case.rope_tail} "
          f"fdt={case.freq_dtype} cache={[c.dtype for c in case.caches]} q={case.q_dtype} "
          f"T={case.T} B={case.batch} knobs={kn}", flush=True)
    res = oracle.run_case(case)
    dc = gh.upload(case)
    gh.run(dc)
    torch.cuda.synchronize()
    parity.compare(case, dc, res)

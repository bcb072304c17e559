#!/usr/bin/env python3
"""Throughput of the fused ragged RoPE + split + paged-KV store on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload prefill|decode|dual|radd|bshd|...]

A step is one call of the pass over one batch of seeded synthetic input that
is already resident in HBM.  The default workload is the Llama-3-8B-shaped
prefill (32 Q / 8 KV heads, head_dim 128, bf16, half-split RoPE, theta 5e5,
batch 8 with lengths U[128, 2048], page 128, 32 layers, layer 17).  Other
workloads (decode, dual band, radd, padded continuous batching) are for
measuring the other operations; `gemv_norm` measures the fused GEMV +
partial RMSNorm (one bf16 row of 7168 into 1536 normed and 576 passed-through
columns), a kernel of its own.

The default warm-up (300 launches) is long on purpose: the first few
hundred launches over multi-GB pools run a few per cent slower (clocks and
address-translation warm-up); the timed region measures steady state.

Each step runs on its own set of buffers, cycling through enough sets that
the data touched between two uses of a set exceeds the 256 MB Infinity
Cache: every step reads its inputs from HBM, not from a warm cache.  Each
set is its own seeded batch (seeds s, s+100, s+200, ...), so the steps sample
the workload's length distribution instead of repeating one draw.

Also measured in the same run, just before the timed region: a plain
streaming copy moving the same bytes (half read, half written) -- the
practical bandwidth ceiling at this size.

Printed: one JSON line.  `value` is effective GB/s (algorithmic bytes per
step / wall time per step), `roofline.achieved` the same bytes over the
kernel's own average duration (HIP events around the timed launches on the
launch stream), `kernel_us` that average and the p10/p50/p90 of single
launches (each between its own events), `cpu_baseline` the CPU oracle on the
host, single-threaded.  The default (prefill) line also carries `decode`:
the Llama-3-8B-shaped decode workload (256 sequences of one new token),
measured first with its own launch counts (--decode-steps, --decode-warmup)
and its own same-size copy ceiling.  `roofline.traffic` and `tcc_hit_rate`
come from the committed counter summary under profiles/ while its kernel
source hash matches the sources built.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective HBM GB/s & tokens/s of fused RoPE+paged-store; % of HBM peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
MALL_BYTES = 256 << 20         # Infinity Cache
KERNEL_NAME = "band_kernel"
KERNEL_SOURCES = ("qk_rope_paged_amd/csrc/band_kernel.hpp", "qk_rope_paged_amd/csrc/kernels.hip",
                  "qk_rope_paged_amd/csrc/kernels_fp8.hip", "qk_rope_paged_amd/csrc/kernels_qout.hip",
                  "qk_rope_paged_amd/csrc/kernels_pack.hip", "qk_rope_paged_amd/csrc/kernels_mixed.hip",
                  "qk_rope_paged_amd/csrc/engine.hpp",
                  "qk_rope_paged_amd/csrc/abi.cpp")
# the fused GEMV + partial RMSNorm (MatmulFusedPartialRMSNorm page): its own
# kernel, sources and workloads
GEMV_KERNEL_NAME = "gemv_norm_kernel"
GEMV_SOURCES = ("qk_rope_paged_amd/csrc/gemv_norm.hip", "qk_rope_paged_amd/csrc/gemv_norm.hpp",
                "qk_rope_paged_amd/csrc/abi_gemv.cpp")
GEMV_WORKLOADS = ("gemv_norm", "gemv_norm_rows4", "gemv_norm_t")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _code_only(text: str) -> str:
    """C/C++ source without comments, trailing blanks and blank lines (string
    and character literals kept as they are)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    lines = (ln.rstrip() for ln in "".join(out).split("\n"))
    return "\n".join(ln for ln in lines if ln)


def kernel_name(workload: str) -> str:
    if workload == "gemv_norm_t":
        return "gemv_norm_t_kernel"     # W stored [k][n]
    return GEMV_KERNEL_NAME if workload in GEMV_WORKLOADS else KERNEL_NAME


def kernel_source_hash(sources=None) -> str:
    """Hash of the code of the kernel sources: a counter summary taken on the
    same code stays valid across edits of comments."""
    h = hashlib.sha256()
    for rel in sources or KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def source_hash_for(workload: str) -> str:
    return kernel_source_hash(GEMV_SOURCES if workload in GEMV_WORKLOADS else None)


def _traffic_summary(workload: str):
    """Key/value lines of the committed counter summary of this workload, or
    None when it is missing or was taken from a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"{kernel_name(workload)}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.split("#")[0].strip()
    if kv.get("kernel_source_sha256") != source_hash_for(workload):
        return None
    return kv


def tcc_hit_rate_from_profiles(workload: str):
    """TCC hit rate (TCC_HIT / (TCC_HIT + TCC_MISS)) of the kernel on this
    workload from the committed counter summary, or None (missing or stale)."""
    kv = _traffic_summary(workload)
    try:
        return None if kv is None else float(kv["tcc_hit_rate"])
    except (KeyError, ValueError):
        return None


def traffic_from_profiles(workload: str, seeds):
    """Measured HBM bytes per launch, averaged like the timed steps, from the
    committed counter summary (per-batch read and write bytes, already scaled
    by the copy calibration), or None when the summary is missing, lacks a
    batch, or was taken from a different kernel source."""
    kv = _traffic_summary(workload)
    if kv is None:
        return None
    total = 0.0
    try:
        for sd in seeds:
            rd, wr = kv[f"seed_{sd}_bytes"].split()[:2]
            total += float(rd) + float(wr)
    except (KeyError, ValueError):
        return None
    return int(total / len(seeds))


def algorithmic_bytes(case) -> int:
    """Bytes the operation must move: inputs read, outputs written, cache rows
    read for in-place updates, distinct freqs rows, metadata and gammas."""
    import numpy as np
    from synth import cases as sc

    eb = sc.ELEM_BYTES[case.dtype]
    if case.op == "gemv_norm":   # x and W read, gamma read, every output written
        return eb * (case.m * case.k + case.n * case.k + case.n_normed + case.m * case.n)
    qeb = sc.ELEM_BYTES[case.q_dtype]
    T = case.T
    seq, pos = cache_rows(case)

    def row(c):   # bytes of one cache head row (an FP8 row carries its scale)
        return c.head_dim * sc.ELEM_BYTES[c.dtype] + (
            sc.ELEM_BYTES[c.scale_dtype] if c.dtype == sc.FP8 else 0)

    total = 0
    if case.op == "bshd":
        c = case.caches[0]
        D, Hk, Hq = c.head_dim, c.num_kv_heads, case.n_q_heads
        total += 2 * T * Hq * D * eb                 # every q_proj row read and written
        total += 2 * len(pos) * Hk * row(c)          # real rows: K read and written in place
    elif case.op == "store":
        c = case.caches[0]
        D, Hk, Hq = c.head_dim, c.num_kv_heads, case.n_q_heads
        total += T * (Hq + 2 * Hk) * D * eb          # qkv read
        total += T * Hq * D * qeb                    # q_out written
        total += T * 2 * Hk * row(c)                 # K and V rows written
    elif case.op in ("norm", "dual"):
        for b in case.bands:
            c = case.caches[b.cache]
            D, Hk = c.head_dim, c.num_kv_heads
            total += 2 * T * b.n_q_heads * D * eb    # Q read + written
            total += T * Hk * (D * eb if b.k_col >= 0 else row(c))   # K read (buffer or cache)
            total += T * Hk * row(c)                 # K written
            if b.v_col >= 0:
                total += T * Hk * (D * eb + row(c))  # V read + written
            total += (int(b.q_gamma is not None) + int(b.k_gamma is not None)) * D * eb
    elif case.op == "radd":
        c = case.caches[0]
        rows = T * 2 * c.num_kv_heads
        total += rows * (c.head_dim * eb + 2 * row(c))   # read a, read cache, write cache
    if case.freqs is not None and len(pos):
        total += len(np.unique(pos)) * case.rope_dim * sc.ELEM_BYTES[case.freq_dtype]
    total += (case.batch + (0 if case.op == "bshd" else 1)) * 4   # offsets / valid lengths
    for c in case.caches:
        total += case.batch * 4                                    # cache lengths
        if len(pos):                                               # distinct page-table entries
            total += len(np.unique(seq * (c.max_pages_per_seq + 1) + pos // c.page_size)) * 4
    return int(total)


def cache_rows(case):
    """(sequence, cache position) of every row that reaches the cache: every
    token of a ragged op; the rows below their sequence's valid length on the
    padded grid.  A position is the sequence's cache length plus the row's
    index within the sequence."""
    import numpy as np

    off = case.offsets.astype(np.int64)
    seqs, out = [], []
    for b in range(case.batch):
        n = int(off[b + 1] - off[b])
        if case.op == "bshd":
            n = min(n, int(case.lengths[b]))
        cl = int(case.caches[0].cache_lengths[b + case.batch_offset])
        out.append(np.arange(cl, cl + n))
        seqs.append(np.full(n, b, np.int64))
    if not out:
        return np.zeros(0, np.int64), np.zeros(0, np.int64)
    return np.concatenate(seqs), np.concatenate(out)


def case_tokens(case) -> int:
    """Tokens a step processes (the padded grid counts its real rows only;
    the GEMV its input rows)."""
    if case.op == "gemv_norm":
        return case.m
    return len(cache_rows(case)[1]) if case.op == "bshd" else case.T


DEFAULT_SEED = {"prefill": 2, "decode": 3, "dual": 4, "radd": 5, "bshd": 6, "prefill_tp8": 2,
                "decode_tp8": 3, "dual_tp8": 4}
DEFAULT_SEED.update({f"{k}_fp8": v for k, v in list(DEFAULT_SEED.items())})
DEFAULT_SEED["gemv_norm"] = DEFAULT_SEED["gemv_norm_rows4"] = DEFAULT_SEED["gemv_norm_t"] = 7


def make_case(workload: str, seed: int = None):
    from synth import cases as sc
    fn = sc.GEMV_WORKLOADS[workload] if workload in GEMV_WORKLOADS else sc.WORKLOADS[workload]
    return fn(seed=DEFAULT_SEED[workload] if seed is None else seed)


def workload_config(case, cases) -> dict:
    from synth import cases as sc
    if case.op == "gemv_norm":
        return {"workload": "matmul_fused_partial_rmsnorm:" + case.name, "rows": case.m,
                "k": case.k, "n": case.n, "n_normed": case.n_normed,
                "weights": "W [n][k] N(0, 1/k), x N(0, 1), gamma N(1, 0.1)",
                "seeds": [x.seed for x in cases]}
    c = case.caches[0]
    cfg = {"workload": {"store": "rope_split_store_paged", "norm": "qk_rmsnorm_rope_paged",
                        "dual": "dual_band", "radd": "kv_cache_radd",
                        "bshd": "fused_qk_rope_bshd_continuous_batch"}[case.op] + ":" + case.name,
           "batch": case.batch, "head_dim": c.head_dim, "kv_heads": c.num_kv_heads,
           "page_size": c.page_size, "num_layers": c.num_layers, "layer_idx": case.layer_idx,
           "seeds": [x.seed for x in cases], "tokens_per_batch": [x.T for x in cases],
           "tokens_mean": round(sum(x.T for x in cases) / len(cases), 1)}
    if case.op in ("store", "bshd"):
        cfg["q_heads"] = case.n_q_heads
    if any(x.dtype == sc.FP8 for x in case.caches):
        cfg["kv_cache"] = "fp8 e4m3, " + case.caches[0].scale_dtype + " scale per row"
    if case.op == "bshd":
        cfg["seq_len"] = case.seq_len
        cfg["real_tokens_per_batch"] = [case_tokens(x) for x in cases]
        cfg["freq_dtype"] = case.freq_dtype
    if case.op in ("store", "norm", "dual", "bshd"):
        cfg["rope"] = "interleaved" if case.interleaved else "half-split"
        cfg["rope_dim"] = case.rope_dim
    if case.op == "dual":
        cfg["q_heads"] = [b.n_q_heads for b in case.bands]
    if case.op == "radd":
        cfg["batch_offset"] = case.batch_offset
    return cfg


def build_sets(cases, share_freqs: bool = True):
    """One device copy per case.  Store-op pools larger than 2 GiB are shared:
    every set after the first gets a page table whose referenced entries
    point at fresh pages, disjoint from the pages any other set touches, so
    no set overwrites another's rows.  With `share_freqs`, sets whose freqs
    table equals the first set's use that one device table: a model's
    freqs_cis is one buffer read by every layer at every step, while the
    batches' own inputs, caches and metadata stay separate (and cold)."""
    import numpy as np
    import torch
    from tests import gpu_harness as gh

    def referenced(case):
        c = case.caches[0]
        seq = np.repeat(np.arange(case.batch), np.diff(case.offsets.astype(np.int64)))
        pidx = cache_rows(case)[1] // c.page_size
        return np.unique(seq * c.max_pages_per_seq + pidx)

    first = cases[0]
    sets = [gh.upload(first)]
    shared = first.op == "store" and first.caches[0].nbytes > (2 << 30)
    if shared:
        c0 = first.caches[0]
        used = np.unique(c0.lookup_table.reshape(-1)[referenced(first)].astype(np.int64))
        free = np.setdiff1d(np.arange(c0.num_pages), used)
        cursor = 0
    for case in cases[1:]:
        if not shared:
            sets.append(gh.upload(case))
            continue
        host = case.caches[0]
        entries = referenced(case)
        if cursor + len(entries) > len(free):
            raise RuntimeError("pool too small for disjoint buffer sets")
        tab = np.full(host.lookup_table.size, 0xFFFFFFFF, dtype=np.uint32)
        tab[entries] = free[cursor:cursor + len(entries)]
        cursor += len(entries)
        saved = case.caches
        case.caches = []
        dc = gh.upload(case)
        case.caches = saved
        base = sets[0].caches[0]
        ttab = torch.from_numpy(tab.view(np.int32)).cuda()
        lens = torch.from_numpy(host.cache_lengths.astype(np.uint32).view(np.int32)).cuda()
        desc = gh.qrp.PagedCache(**{**base.desc.__dict__, "lookup_table": ttab,
                                    "cache_lengths": lens})
        dc.caches = [gh.DeviceCache(host=host, pool=base.pool, cache_lengths=lens,
                                    lookup_table=ttab, desc=desc)]
        sets.append(dc)
    if share_freqs and first.freqs is not None:
        for dc, case in zip(sets[1:], cases[1:]):
            if case.freq_dtype == first.freq_dtype and np.array_equal(case.freqs, first.freqs):
                dc.freqs = sets[0].freqs
    return sets, shared


def time_launches(calls, steps: int, warmup: int):
    """Warm up, then time `steps` launches cycling through `calls`: wall time
    between two synchronisations, and each launch's duration from events
    recorded around it on the launch stream."""
    import torch

    for i in range(warmup):
        calls[i % len(calls)]()
    torch.cuda.synchronize()
    ev_s = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ev_e = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        ev_s[k].record()
        calls[k % len(calls)]()
        ev_e[k].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, [s.elapsed_time(e) / 1e3 for s, e in zip(ev_s, ev_e)]


def time_region(calls, steps: int, warmup: int):
    """Warm up, then run `steps` launches back to back (cycling `calls`)
    between one pair of HIP events on the launch stream and two
    synchronisations: (wall seconds, GPU seconds)."""
    import torch

    for i in range(warmup):
        calls[i % len(calls)]()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for k in range(steps):
        calls[k % len(calls)]()
    ev1.record()
    torch.cuda.synchronize()
    return time.perf_counter() - t0, ev0.elapsed_time(ev1) / 1e3


def time_graph(launchers, steps: int, max_nodes: int = 250, wall_out=None) -> float:
    """Average GPU seconds per launch when the launches are replayed from a
    HIP graph: min(steps, max_nodes) launches (cycling `launchers`, each a
    function of the stream to launch on) are captured once and the graph is
    replayed until `steps` launches have run, between one pair of events
    (and two synchronisations: their wall time goes to `wall_out[0]`).
    Launch-bound kernels are issued this way in a serving loop; the host's
    per-launch cost then drops out of the measurement."""
    import torch

    n = min(steps, max_nodes)
    reps = -(-steps // n)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(min(3, len(launchers))):
            launchers[i](s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for k in range(n):
            launchers[k % len(launchers)](s)
    torch.cuda.synchronize()
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(reps):
        g.replay()
    ev1.record()
    torch.cuda.synchronize()
    if wall_out is not None:
        wall_out[0] = time.perf_counter() - t0
    del g
    return ev0.elapsed_time(ev1) / 1e3 / (reps * n)


def copy_ceiling(nbytes: int, n_bufs: int, steps: int, graph: bool = False) -> dict:
    """A plain streaming copy of nbytes/2 (read) into nbytes/2 (written),
    cycling through n_bufs buffer pairs: the best of 1, 2, 4 and 8
    chunks/thread;
    with `graph`, the launches are replayed from a HIP graph."""
    import ctypes
    import torch
    from qk_rope_paged_amd import build as hip_build

    lib = ctypes.CDLL(hip_build.COPY_LIB_PATH)
    lib.qrp_bench_stream_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64,
                                          ctypes.c_int32, ctypes.c_void_p]
    lib.qrp_bench_stream_copy.restype = ctypes.c_int32
    half = (nbytes // 2) // 16 * 16
    bufs = [(torch.ones(half // 8, dtype=torch.int64, device="cuda"),
             torch.empty(half // 8, dtype=torch.int64, device="cuda")) for _ in range(n_bufs)]
    stream = torch.cuda.current_stream().cuda_stream
    best = None
    for u in (1, 2, 4, 8):
        def mk(a, b, u=u):
            def f():
                if lib.qrp_bench_stream_copy(b.data_ptr(), a.data_ptr(), half, u, stream) != 0:
                    raise RuntimeError("copy launch failed")
            return f
        if graph:
            def mkg(a, b, u=u):
                def f(st):
                    if lib.qrp_bench_stream_copy(b.data_ptr(), a.data_ptr(), half, u,
                                                 st.cuda_stream) != 0:
                        raise RuntimeError("copy launch failed")
                return f
            time_region([mk(a, b) for a, b in bufs], 10, 10)
            avg = time_graph([mkg(a, b) for a, b in bufs], steps)
        else:
            _, gpu = time_region([mk(a, b) for a, b in bufs], steps, 10)
            avg = gpu / steps
        if best is None or avg < best[1]:
            best = (u, avg)
    ok = all(torch.equal(a, b) for a, b in bufs[:2])
    del bufs
    torch.cuda.empty_cache()
    return {"value": round(2 * half / best[1] / 1e9, 2), "unit": "GB/s",
            "kernel_us": round(best[1] * 1e6, 3), "bytes": 2 * half,
            "chunks_per_thread": best[0], "verified": ok,
            "kind": "nontemporal streaming copy, same bytes as one step (half read, half written)"
                    + (", launches replayed from a HIP graph" if graph else "")}


def cpu_baseline(cases, seconds: float, max_passes: int) -> dict:
    """The CPU oracle as it stands, single-threaded, on the same batches
    (cycled), repeated until about `seconds` of oracle time."""
    import oracle

    total, passes, nbytes, ntok = 0.0, 0, 0, 0
    while passes < max_passes and (passes == 0 or total < seconds):
        case = cases[passes % len(cases)]
        res = oracle.run_gemv(case, trace=False) if case.op == "gemv_norm" else \
            oracle.run_case(case, trace=False)
        if res.status != 0:
            raise RuntimeError(f"oracle failed with status {res.status}")
        total += res.seconds
        nbytes += algorithmic_bytes(case)
        ntok += case_tokens(case)
        passes += 1
    return {"value": round(nbytes / total / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{passes} full passes over the first {min(passes, len(cases))} seeded "
                      f"batches ({ntok} tokens), {total:.1f} s of oracle time (C call only)",
            "tokens_per_s": round(ntok / total, 1),
            "host": {"nproc": os.cpu_count(), "cpu_model": _cpu_model()}}


def _cpu_model() -> str:
    """The host CPU's model name, from /proc/cpuinfo (empty where it is absent)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def check_parity(case, dc, shared_pool: bool) -> str:
    """Part of the CPU-baseline leg: the oracle that leg times also checks the
    first device set (store ops and the GEMV repeat to the same result;
    in-place ops accumulate, so they are not checked here).  With a shared
    pool the other sets' pages are not expected to hold the sentinel."""
    if case.op == "gemv_norm":
        import oracle
        from tests import gemv_parity
        from tests import gpu_harness as gh
        res = oracle.run_gemv(case)
        gemv_parity.check(case, res, gh.to_numpy_bits(dc.normed, case.dtype),
                          gh.to_numpy_bits(dc.unnormed, case.dtype))
        return "ok"
    if case.op != "store":
        return "not checked (in-place op applied repeatedly)"
    import oracle
    from tests import parity
    res = oracle.run_case(case)
    parity.compare(case, dc, res, untouched_pages=not shared_pool)
    return "ok"


def percentiles(values, qs=(10, 50, 90)):
    """Nearest-rank percentiles of a list."""
    v = sorted(values)
    return {q: v[min(len(v) - 1, (q * len(v)) // 100)] for q in qs}


def prepare(workload: str, base_seed: int, sets_arg: int, share_freqs: bool = True):
    """Seeded batches of the workload and their device buffer sets."""
    import torch
    from tests import gpu_harness as gh

    t_gen = time.perf_counter()
    first = make_case(workload, base_seed)
    per_step = max(algorithmic_bytes(first), 1)
    n_sets = sets_arg or min(16, max(2, -(-3 * MALL_BYTES // per_step) + 1))
    cases = [first] + [make_case(workload, base_seed + 100 * k) for k in range(1, n_sets)]
    set_bytes = [algorithmic_bytes(c) for c in cases]
    log(f"[bench] {first.name}: {n_sets} seeded batches, tokens {[c.T for c in cases]}, "
        f"mean bytes/step {sum(set_bytes) / n_sets:.0f} (generated in "
        f"{time.perf_counter() - t_gen:.1f}s)")
    if first.op == "gemv_norm":
        sets, shared_pool = [gh.upload_gemv(c) for c in cases], False
        calls = [gh.run_gemv(dg, prepare=True) for dg in sets]
    else:
        sets, shared_pool = build_sets(cases, share_freqs)
        calls = [gh.run(dc, prepare=True) for dc in sets]
    torch.cuda.synchronize()
    return cases, set_bytes, sets, shared_pool, calls


def measure(workload: str, calls, cases, set_bytes, steps: int, warmup: int,
            launchers=None) -> dict:
    """K launches back to back (cycling the sets) between one pair of HIP
    events on the launch stream, then the same K launches each between its
    own pair (the spread of single launches; an event pair adds about 2 us
    to what it measures).  With `launchers`, the timed K launches are
    replayed from a HIP graph instead (after W eager warm-up launches)."""
    n_sets = len(cases)
    if launchers is None:
        wall, gpu_time = time_region(calls, steps, warmup)
    else:
        import torch
        for i in range(warmup):
            calls[i % n_sets]()
        torch.cuda.synchronize()
        w = [0.0]
        gpu_time = time_graph(launchers, steps, max_nodes=steps, wall_out=w) * steps
        wall = w[0]
    _, durs = time_launches(calls, steps, 0)
    step_bytes = [set_bytes[k % n_sets] for k in range(steps)]
    step_tokens = [case_tokens(cases[k % n_sets]) for k in range(steps)]
    us = percentiles([d * 1e6 for d in durs])
    rate = percentiles([b / d / 1e9 for b, d in zip(step_bytes, durs)])
    achieved = sum(step_bytes) / gpu_time / 1e9
    log(f"[bench] {cases[0].name}: {steps} steps, wall {wall * 1e3:.2f} ms, events "
        f"{gpu_time * 1e3:.2f} ms ({gpu_time / steps * 1e6:.2f} us per launch); single launches "
        f"p10/p50/p90 {us[10]:.2f}/{us[50]:.2f}/{us[90]:.2f} us")
    return {"wall": wall, "gpu_time": gpu_time, "step_bytes": step_bytes,
            "step_tokens": step_tokens, "achieved": achieved,
            "kernel_us": {"avg": round(gpu_time / steps * 1e6, 3),
                          "single_launch_p10": round(us[10], 3),
                          "single_launch_p50": round(us[50], 3),
                          "single_launch_p90": round(us[90], 3)},
            "single_launch_gbs": {"p10": round(rate[10], 1), "p50": round(rate[50], 1),
                                  "p90": round(rate[90], 1)},
            "traffic": traffic_from_profiles(workload, [cases[k % n_sets].seed
                                                        for k in range(steps)]),
            "tcc_hit_rate": tcc_hit_rate_from_profiles(workload)}


def graph_launchers(sets, gemv: bool):
    """One launcher per buffer set, taking the stream to launch on."""
    from tests import gpu_harness as gh
    if gemv:
        return [lambda st, dg=dg: gh.run_gemv(dg, stream=st) for dg in sets]
    return [lambda st, dc=dc: gh.run(dc, stream=st) for dc in sets]


def decode_block(args) -> dict:
    """The Llama-3-8B-shaped decode workload (256 sequences of one new token),
    measured with its own launch counts and copy ceiling: the second
    configuration the fused kernel is held to.  One decode launch takes less
    GPU time than the host needs to issue it (a few microseconds through
    the C ABI), so eagerly issued launches measure the host; the kernel's
    rate comes from launches replayed from a HIP graph, the way a serving
    loop issues them, and the copy ceiling is measured the same way.  The
    eager figures are kept beside it."""
    import torch

    w = "decode"
    cases, set_bytes, sets, _, calls = prepare(w, DEFAULT_SEED[w], 0, not args.per_set_freqs)
    m = measure(w, calls, cases, set_bytes, args.decode_steps, args.decode_warmup)
    per_launch = time_graph(graph_launchers(sets, False), args.decode_steps)
    del sets, calls
    torch.cuda.empty_cache()
    n = len(cases)
    mean_bytes = sum(set_bytes) / n
    achieved = mean_bytes / per_launch / 1e9
    cc = copy_ceiling(int(mean_bytes), n, max(200, args.decode_steps), graph=True)
    log(f"[bench] decode: graph replay {per_launch * 1e6:.3f} us per launch, copy "
        f"{cc['kernel_us']:.3f} us")
    return {"workload": workload_config(cases[0], cases)["workload"], "sequences": cases[0].batch,
            "steps": args.decode_steps, "warmup": args.decode_warmup,
            "kernel_us": {"graph_replay_avg": round(per_launch * 1e6, 3),
                          "eager_avg": m["kernel_us"]["avg"],
                          "eager_single_launch_p10": m["kernel_us"]["single_launch_p10"],
                          "eager_single_launch_p50": m["kernel_us"]["single_launch_p50"],
                          "eager_single_launch_p90": m["kernel_us"]["single_launch_p90"]},
            "achieved": round(achieved, 2), "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "eager_achieved": round(m["achieved"], 2),
            "tokens_per_s": round(case_tokens(cases[0]) / per_launch, 1),
            "algorithmic_bytes_per_step": round(mean_bytes),
            "copy_ceiling": {"value": cc["value"], "kernel_us": cc["kernel_us"],
                             "kind": cc["kind"]},
            "frac_of_copy_ceiling": round(achieved / cc["value"], 4),
            "traffic": m["traffic"], "tcc_hit_rate": m["tcc_hit_rate"]}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default="prefill",
                    choices=["prefill", "decode", "dual", "radd", "bshd", "prefill_fp8",
                             "decode_fp8", "dual_fp8", "radd_fp8", "bshd_fp8", "prefill_tp8",
                             "decode_tp8", "dual_tp8", *GEMV_WORKLOADS])
    ap.add_argument("--sets", type=int, default=0, help="buffer sets to cycle (0: auto)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--cpu-max-passes", type=int, default=30)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--no-copy-ceiling", action="store_true")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode block of the default (prefill) line")
    ap.add_argument("--per-set-freqs", action="store_true",
                    help="give every buffer set its own copy of the freqs table (default: the "
                         "sets share one, as a model's layers do)")
    ap.add_argument("--graph", action="store_true",
                    help="replay the timed launches from a HIP graph (captured before "
                         "the timed region)")
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--decode-warmup", type=int, default=300)
    ap.add_argument("--seed", type=int, default=None, help="seed of the first batch")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run a plain device copy of this size first (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the pass shards by sequence or by head with "
              "no exchange between GPUs, and this library has no multi-GPU code. "
              "Run with --gpus 1.", file=sys.stderr)
        return 2

    from qk_rope_paged_amd import build as hip_build
    if not os.path.exists(hip_build.LIB_PATH):
        hip_build.build()
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)

    # The default line also carries the decode configuration, measured
    # first, on its own buffers.
    decode = None
    if args.workload == "prefill" and not args.no_decode:
        decode = decode_block(args)

    base_seed = args.seed if args.seed is not None else DEFAULT_SEED[args.workload]
    cases, set_bytes, sets, shared_pool, calls = prepare(args.workload, base_seed, args.sets,
                                                         not args.per_set_freqs)
    first = cases[0]
    n_sets = len(cases)

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: 3 copies of {n} bytes")
        del src, dst

    K = args.steps
    # The copy ceiling (a plain copy of one step's mean bytes, replayed from
    # a HIP graph when the timed launches are) is measured just before the
    # timed region: the GPU has idled while the batches were
    # generated on the host, and this brings it back to its steady clock
    # before the W warm-up steps, as a serving loop that runs continuously
    # would find it.
    cc = None
    if not args.no_copy_ceiling:
        log("[bench] timing the copy ceiling ...")
        cc_bytes = sum(set_bytes[k % n_sets] for k in range(K)) / K
        cc = copy_ceiling(int(cc_bytes), n_sets, max(20, K // 2), graph=args.graph)

    # Timed region: K steps back to back on the launch stream, bracketed by
    # one pair of HIP events (GPU time) and two synchronisations (wall time).
    launchers = graph_launchers(sets, first.op == "gemv_norm") if args.graph else None
    m = measure(args.workload, calls, cases, set_bytes, K, args.warmup, launchers)
    wall, gpu_time = m["wall"], m["gpu_time"]

    # the oracle runs only in the CPU-baseline leg: its first batch also
    # checks the GPU's outputs
    parity_status = "not checked (no CPU-baseline leg)"
    cpu = None
    if not args.no_cpu_baseline:
        if not args.no_parity:
            parity_status = check_parity(first, sets[0], shared_pool)
            log(f"[bench] parity: {parity_status}")
        log("[bench] timing the CPU oracle ...")
        cpu = cpu_baseline(cases, args.cpu_seconds, args.cpu_max_passes)

    mean_bytes = sum(m["step_bytes"]) / K
    value = sum(m["step_bytes"]) / wall / 1e9
    achieved = m["achieved"]
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall / K * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": first.dtype,
        "data": "synthetic (seeded batches with the workload's shapes and length distribution)",
        "config": {**workload_config(first, cases),
                   **({} if first.op == "gemv_norm" else
                      {"freqs_table": "one copy per batch" if args.per_set_freqs else
                       "one table shared by every batch"})},
        "tokens_per_s": round(sum(m["step_tokens"]) / wall, 1),
        "hbm_peak_frac": round(value / HBM_PEAK_GBS, 4),
        "algorithmic_bytes_per_step": round(mean_bytes),
        "kernel_us": m["kernel_us"],
        "timed_launches": "replayed from a HIP graph" if args.graph else "issued eagerly",
        "single_launch_gbs": m["single_launch_gbs"],
        "parity": parity_status,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": m["traffic"], "tcc_hit_rate": m["tcc_hit_rate"],
                     "kernel": kernel_name(args.workload)},
    }
    if cc is not None:
        out["copy_ceiling"] = cc
        out["roofline"]["frac_of_copy_ceiling"] = round(achieved / cc["value"], 4)
    if decode is not None:
        out["decode"] = decode
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

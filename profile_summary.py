#!/usr/bin/env python3
"""Turn rocprofv3 output databases into the short text summaries kept under
profiles/.

    # kernel durations (from `rocprofv3 --kernel-trace --stats -d DIR -- python bench.py ...`)
    python profile_summary.py trace DIR --label "..." --command "..."

    # SQ counters per dispatch (one `rocprofv3 --pmc SQ_...` run)
    python profile_summary.py counters DIR --workload gemv_norm --command "..."

    # HBM traffic per launch (from three `rocprofv3 --pmc ...` runs of
    # `bench.py --steps N --warmup 0 --sets N --copy-calibration-mib M ...`)
    python profile_summary.py traffic --fetch DIR --write DIR --tcc DIR \\
        --workload prefill --sets N --calib-mib M --command "..."

FETCH_SIZE and WRITE_SIZE are scaled by what they read for the calibration
copy of M MiB in the same run (a copy of M MiB reads and writes exactly M MiB).
The band kernel's dispatches are matched to the bench's batches in launch
order: launch i ran buffer set i mod N, whose batch has seed s + 100 (i mod N).
Only the standard library and the synthetic-input generator are used.
"""
from __future__ import annotations

import argparse
import glob
import os
import sqlite3
import statistics
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BAND = "band_kernel"
CALIB = "__amd_rocclr_copyBuffer"


def _db(path: str) -> sqlite3.Connection:
    files = sorted(glob.glob(os.path.join(path, "**", "*.db"), recursive=True))
    if not files:
        raise SystemExit(f"no rocprofv3 database under {path}")
    return sqlite3.connect(files[0])


def trace(args) -> str:
    con = _db(args.dir)
    rows = list(con.execute("select name, duration, grid_x, workgroup_x, vgpr_count, sgpr_count, "
                            "lds_size from kernels order by start"))
    by = {}
    for name, dur, gx, wx, vg, sg, lds in rows:
        by.setdefault(name, []).append((dur, gx, wx, vg, sg, lds))
    out = [f"# Kernel trace: {args.label}", "",
           f"Command: `{args.command}`", "",
           "Durations in microseconds (rocprofv3 kernel trace).", "",
           "| kernel | calls | avg | median | min | max |", "|---|---|---|---|---|---|"]
    for name, v in sorted(by.items(), key=lambda kv: -sum(x[0] for x in kv[1])):
        d = [x[0] / 1e3 for x in v]
        out.append(f"| `{name[:110]}` | {len(d)} | {statistics.mean(d):.2f} | "
                   f"{statistics.median(d):.2f} | {min(d):.2f} | {max(d):.2f} |")
    kern = args.kernel
    band = [(k, v) for k, v in by.items() if kern in k]
    if args.warmup is not None and args.steps:
        # every band-kernel launch in launch order: batches whose waves hold
        # one pass run the one-pass build, so one run can use two builds.
        # With --graph the bench replays its K timed launches from a HIP
        # graph: after the W warm-up launches come 3 eager launches, two
        # untimed replays (2K launches), then the K timed ones.
        seq = [dur for name, dur, *_ in rows if kern in name]
        first = args.warmup + (3 + 2 * args.steps if args.graph else 0)
        timed = [d / 1e3 for d in seq[first:first + args.steps]]
        names = ", ".join(f"`{k[:60]}...`" for k, _ in band)
        out += ["", f"Timed region of the bench ({kern} launches {first} to "
                    f"{first + len(timed) - 1}, of {names}"
                    f"{', replayed from a HIP graph' if args.graph else ''}): "
                    f"average {statistics.mean(timed):.2f} us, median "
                    f"{statistics.median(timed):.2f} us over {len(timed)} launches."]
    for name, v in band:
        out += ["", f"`{name}`: LDS {v[0][5]} bytes, {v[0][2]} threads per block.", "",
                "| grid threads (one batch) | launches | avg us | min us |", "|---|---|---|---|"]
        grids = {}
        for dur, gx, *_ in v:
            grids.setdefault(gx, []).append(dur / 1e3)
        for gx, d in sorted(grids.items()):
            out.append(f"| {gx} | {len(d)} | {statistics.mean(d):.2f} | {min(d):.2f} |")
    return "\n".join(out) + "\n"


def _pmc(path: str):
    con = _db(path)
    return list(con.execute("select dispatch_id, name, counter_name, counter_value from pmc_events "
                            "order by dispatch_id"))


def _per_kernel(rows, counter, kern=BAND):
    band, calib = [], []
    for did, name, cn, cv in rows:
        if cn != counter:
            continue
        if kern in name:
            band.append(cv)
        elif name == CALIB:
            calib.append(cv)
    return band, calib


def traffic(args) -> str:
    import bench

    calib_kib = args.calib_mib * 1024
    kern = bench.kernel_name(args.workload)
    fb, fc = _per_kernel(_pmc(args.fetch), "FETCH_SIZE", kern)
    wb, wc = _per_kernel(_pmc(args.write), "WRITE_SIZE", kern)
    tcc = _pmc(args.tcc)
    hits, _ = _per_kernel(tcc, "TCC_HIT_sum", kern)
    miss, _ = _per_kernel(tcc, "TCC_MISS_sum", kern)
    # the calibration copy is the largest copyBuffer dispatch(es)
    fcal = [v for v in fc if v > 0.25 * calib_kib]
    wcal = [v for v in wc if v > 0.5 * calib_kib]
    if not fcal or not wcal:
        raise SystemExit("calibration copy not found")
    fscale = calib_kib / statistics.median(fcal)
    wscale = calib_kib / statistics.median(wcal)
    base = bench.DEFAULT_SEED[args.workload] if args.seed is None else args.seed
    seeds = [base + 100 * k for k in range(args.sets)]
    per = {}
    for i, (f, w) in enumerate(zip(fb, wb)):
        per.setdefault(seeds[i % args.sets], []).append((f * 1024 * fscale, w * 1024 * wscale))
    hit_rate = [h / (h + m) for h, m in zip(hits, miss) if h + m > 0]
    lines = [f"# HBM traffic of {kern} on the {args.workload} workload "
             f"(rocprofv3 PMC, one line per seeded batch)",
             f"# command: {args.command}",
             f"# calibration: a {args.calib_mib} MiB device copy in the same run read "
             f"{statistics.median(fcal):.1f} KiB by FETCH_SIZE and wrote "
             f"{statistics.median(wcal):.1f} KiB by WRITE_SIZE; the kernel's counts are "
             f"multiplied by fetch_scale and write_scale",
             f"kernel_source_sha256: {bench.source_hash_for(args.workload)}",
             f"fetch_scale: {fscale:.5f}",
             f"write_scale: {wscale:.5f}"]
    tot_r = tot_w = tot_a = 0.0
    for sd in seeds:
        if sd not in per:
            continue
        r = statistics.mean(x[0] for x in per[sd])
        w = statistics.mean(x[1] for x in per[sd])
        case = bench.make_case(args.workload, sd)
        alg = bench.algorithmic_bytes(case)
        tot_r += r
        tot_w += w
        tot_a += alg
        lines.append(f"seed_{sd}_bytes: {r:.0f} {w:.0f}   # read, written; algorithmic {alg} "
                     f"({(r + w) / alg:.4f}x), T={case.T}")
    n = len([s for s in seeds if s in per])
    lines += [f"fetch_bytes_per_launch: {tot_r / n:.0f}",
              f"write_bytes_per_launch: {tot_w / n:.0f}",
              f"measured_over_algorithmic: {(tot_r + tot_w) / tot_a:.4f}",
              f"tcc_hit_rate: {statistics.mean(hit_rate):.4f}   # TCC_HIT / (TCC_HIT + TCC_MISS), "
              f"mean over {len(hit_rate)} launches"]
    return "\n".join(lines) + "\n"


def counters(args) -> str:
    """Mean of each counter per dispatch of the workload's kernel (SQ
    counters of one `rocprofv3 --pmc` pass)."""
    import bench

    kern = bench.kernel_name(args.workload)
    per = {}
    for did, name, cn, cv in _pmc(args.dir):
        if kern in name:
            per.setdefault(cn, {}).setdefault(did, 0.0)
            per[cn][did] += cv
    lines = [f"# SQ counters of {kern} on the {args.workload} workload (rocprofv3 PMC, mean per "
             f"dispatch)", f"# command: {args.command}",
             f"kernel_source_sha256: {bench.source_hash_for(args.workload)}"]
    for cn in sorted(per):
        lines.append(f"{cn}: {statistics.mean(per[cn].values()):.0f}   # over {len(per[cn])} dispatches")
    return "\n".join(lines) + "\n"


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    sub = ap.add_subparsers(dest="mode", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("--label", required=True)
    t.add_argument("--command", required=True)
    t.add_argument("--warmup", type=int, default=None, help="warm-up launches before the timed region")
    t.add_argument("--steps", type=int, default=0, help="launches in the timed region")
    t.add_argument("--kernel", default=BAND, help="name (or part) of the kernel timed")
    t.add_argument("--graph", action="store_true", help="the bench ran with --graph")
    p = sub.add_parser("traffic")
    p.add_argument("--fetch", required=True)
    p.add_argument("--write", required=True)
    p.add_argument("--tcc", required=True)
    p.add_argument("--workload", required=True)
    p.add_argument("--sets", type=int, required=True)
    p.add_argument("--seed", type=int, default=None)
    p.add_argument("--calib-mib", type=int, required=True)
    p.add_argument("--command", required=True)
    c = sub.add_parser("counters")
    c.add_argument("dir")
    c.add_argument("--workload", required=True)
    c.add_argument("--command", required=True)
    args = ap.parse_args()
    sys.stdout.write({"trace": trace, "traffic": traffic, "counters": counters}[args.mode](args))
    return 0


if __name__ == "__main__":
    sys.exit(main())

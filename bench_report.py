"""Turn benchmark and rocprofv3 output into the text summaries kept under
profiles/ (each summary records the command that produced its input).

  python bench_report.py router   ROUTER_JSON  [--cmd CMD]
  python bench_report.py ceilings CEILINGS_JSON [--cmd CMD]
  python bench_report.py trace    KERNEL_STATS_CSV [--cmd CMD] [--top N]
  python bench_report.py traffic  --fetch CSV --write CSV --kernel SUBSTR --algorithmic BYTES
                                  --workload TEXT --source-sha SHA [--cmd CMD ...]
  python bench_report.py counters COUNTER_CSV [COUNTER_CSV ...] --kernel SUBSTR [--title T] [--workload W]
                                  [--source-sha SHA] [--cmd CMD ...]

ROUTER_JSON / CEILINGS_JSON are the JSON lines printed by `bench.py
--router-sweep` and `bench.py --ceilings`; the CSVs are rocprofv3's
`*_kernel_stats.csv` (from --kernel-trace --stats) and
`*_counter_collection.csv` (from --pmc).  Output goes to stdout.
"""
from __future__ import annotations

import argparse
import csv
import json
import math
import statistics
import sys
from collections import defaultdict


def _last_json(path):
    with open(path) as f:
        lines = [ln for ln in f if ln.strip().startswith("{")]
    return json.loads(lines[-1])


def router(args):
    d = _last_json(args.file)
    ev = d["router_evidence"]
    out = ["# Router evidence: the router's pick against every forced variant", ""]
    out += ["Cache-flushed median per variant (caches flushed by a 1 GiB read before each run), "
            f"{d.get('steps', 30)} runs each, all on one plan per configuration.  "
            "`router / best` = best time / router time (1 = the router picked the fastest; RA-SpMM, abstract: "
            "the router's speed relative to the best kernel per input).  Variants that resolve to the router's "
            "own kernel and launch shape count as the router (their spread is the noise).", ""]
    if args.cmd:
        out += ["Command:", "", "```", *args.cmd, "```", ""]
    out += ["| configuration | reduce | router path | router ms | best ms | best variant | router / best |",
            "|---|---|---|---|---|---|---|"]
    ratios = []
    for cfg, entries in ev.items():
        for e in entries:
            path = next((v.get("path", "") for v in e["variants"] if v["variant"] == "router"), "")
            out.append(f"| {cfg} | {e['reduce']} | {path} | {e['router_ms']:.4f} | {e['best_ms']:.4f} | "
                       f"{e['best_variant']} | {e['router_speed_vs_best']:.3f} |")
            ratios.append(e["router_speed_vs_best"])
    geo = math.exp(sum(math.log(q) for q in ratios) / len(ratios))
    out += ["", f"Geometric mean of router / best over {len(ratios)} configurations: **{geo:.4f}**; "
            f"minimum **{min(ratios):.4f}**.", ""]
    out += [f"Configurations where the router is below {args.detail_below} of the best: the router's pick and "
            f"the {args.top} fastest other variants (the JSON line holds all of them).", ""]
    for cfg, entries in ev.items():
        for e in entries:
            if e["router_speed_vs_best"] >= args.detail_below:
                continue
            out += [f"## {cfg}, {e['reduce']}", "", "| variant | ms | path | route (lanes, vec, F, slices, xcd, nt, "
                    "split, tiles, window) |", "|---|---|---|---|"]
            timed = [v for v in e["variants"] if "ms" in v]
            rest = sorted((v for v in timed if v["variant"] != "router"), key=lambda v: v["ms"])[:args.top]
            for v in [x for x in timed if x["variant"] == "router"] + rest:
                out.append(f"| {v['variant']} | {v['ms']:.4f} | {v['path']} | {v['route']} |")
            out.append("")
    print("\n".join(out))


def ceilings(args):
    d = _last_json(args.file)["ceilings"]
    st = d["stream"]
    out = ["# Bandwidth ceilings of the MI355X", ""]
    if args.cmd:
        out += ["Command:", "", "```", *args.cmd, "```", ""]
    out += [f"Stream ({st['kernels']}, median of {st['reps']} event-timed runs):", "",
            "| read GB/s | write GB/s | copy GB/s (read + write) |", "|---|---|---|",
            f"| {st['read_GBps']} | {st['write_GBps']} | {st['copy_GBps']} |", ""]
    if "read_by_op" in st:
        out += ["Read rate by PyTorch reduction: " + ", ".join(f"{k} {v} GB/s" for k, v in st["read_by_op"].items()),
                ""]
    g = d["gather"]
    out += [f"Random gathers of the row kernel: {g['rows']} rows x {g['deg']} uniform columns over K rows of "
            f"B [K, {g['N']}] fp32, sum; gather bytes nnz * N * 4 = {g['gather_bytes'] / 1e9:.2f} GB per product.", "",
            "| B size MB | K | warm ms | flushed ms | gather GB/s warm | gather GB/s flushed | route |",
            "|---|---|---|---|---|---|---|"]
    for r in g["by_B_size"]:
        out.append(f"| {r['B_MB']} | {r['K']} | {r['warm_ms']:.4f} | {r['flushed_ms']:.4f} | "
                   f"{r['gather_GBps_warm']} | {r['gather_GBps_flushed']} | {r['route']} |")
    print("\n".join(out))


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _col(row, *names):
    low = {k.lower(): v for k, v in row.items()}
    for n in names:
        if n.lower() in low:
            return low[n.lower()]
    raise KeyError(names)


def trace(args):
    rows = _rows(args.file)
    out = ["# Kernel trace", ""]
    if args.cmd:
        out += ["Command:", "", "```", *args.cmd, "```", ""]
    out += ["Durations per dispatch in microseconds.", "",
            "| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
    rows.sort(key=lambda r: -float(_col(r, "TotalDurationNs")))
    for r in rows[:args.top]:
        name = _col(r, "Name")
        name = name if len(name) <= 100 else name[:97] + "..."
        out.append(f"| `{name}` | {_col(r, 'Calls')} | {float(_col(r, 'AverageNs')) / 1e3:.1f} | "
                   f"{float(_col(r, 'MinNs')) / 1e3:.1f} | {float(_col(r, 'MaxNs')) / 1e3:.1f} | "
                   f"{float(_col(r, 'Percentage')):.2f} |")
    print("\n".join(out))


def _per_dispatch(path, counter):
    """{kernel name: [(grid, value per dispatch)]} for one counter."""
    acc = defaultdict(float)
    meta = {}
    for r in _rows(path):
        if _col(r, "Counter_Name") != counter:
            continue
        key = _col(r, "Dispatch_Id", "Correlation_Id")
        acc[key] += float(_col(r, "Counter_Value"))
        meta[key] = (_col(r, "Kernel_Name"), int(float(_col(r, "Grid_Size"))))
    out = defaultdict(list)
    for key, v in acc.items():
        name, grid = meta[key]
        out[name].append((grid, v))
    return out


def _copy_scale(disp, kib_moved):
    """Counter reading of the largest plain device copies against the KiB they
    move: the factor that turns the counter into bytes."""
    copies = [(g, v) for name, xs in disp.items() if "copyBuffer" in name for g, v in xs]
    if not copies:
        return None, None
    copies.sort(key=lambda t: -t[0])
    top = [v for g, v in copies if g == copies[0][0]]
    per = statistics.median(top)
    return kib_moved / per, per


def traffic(args):
    f = _per_dispatch(args.fetch, "FETCH_SIZE")
    w = _per_dispatch(args.write, "WRITE_SIZE")
    gib_kib = 1 << 20
    fs, fper = _copy_scale(f, gib_kib)
    ws, wper = _copy_scale(w, gib_kib)
    if fs is None or ws is None:
        sys.exit("no device copy in the counter runs: run the benchmark with --calibrate-copy")
    out = [f"# HBM traffic of one product, from rocprofv3 hardware counters",
           f"# workload: {args.workload}", "# commands (run from /tmp, repository at $R):"]
    out += [f"#   {c}" for c in args.cmd]
    out += [f"# calibration: a plain 1 GiB device copy reads FETCH_SIZE {fper:.1f} KiB and WRITE_SIZE {wper:.1f} KiB "
            f"per dispatch for {gib_kib} KiB moved each way: FETCH_SIZE x {fs:.4f}, WRITE_SIZE x {ws:.4f}",
            "# per kernel of the product (average over dispatches, KiB per dispatch -> scaled MB):"]
    total = 0.0
    for sub in args.kernel:
        names = [n for n in f if sub in n]
        for n in names:
            fv = statistics.mean(v for _, v in f[n])
            wv = statistics.mean(v for _, v in w.get(n, [(0, 0.0)]))
            rd, wr = fv * fs * 1024, wv * ws * 1024
            total += rd + wr
            out.append(f"#   {n[:90]} grid {f[n][0][0]}: FETCH {fv:.1f} WRITE {wv:.1f} KiB ({len(f[n])} dispatches) "
                       f"-> read {rd / 1e6:.1f} MB, written {wr / 1e6:.1f} MB")
    alg = float(args.algorithmic)
    out += [f"# product total: {total / 1e6:.1f} MB of HBM traffic; algorithmic bytes {alg / 1e6:.1f} MB; "
            f"ratio {total / alg:.3f}",
            f"hbm_bytes_per_launch: {int(total)}", f"algorithmic_bytes_per_launch: {int(alg)}",
            f"fetch_scale: {fs:.4f}", f"write_scale: {ws:.4f}", f"kernel_source_sha: {args.source_sha}"]
    print("\n".join(out))


def counters(args):
    # per file: mean per dispatch of each counter, per kernel; passes of the
    # same kernel (one file each) are merged by kernel name
    merged = defaultdict(lambda: defaultdict(list))
    ndisp = defaultdict(int)
    for path in args.file:
        vals = defaultdict(lambda: defaultdict(float))
        names = {}
        for r in _rows(path):
            kn = _col(r, "Kernel_Name")
            if not any(sub in kn for sub in args.kernel):
                continue
            key = _col(r, "Dispatch_Id", "Correlation_Id")
            vals[key][_col(r, "Counter_Name")] += float(_col(r, "Counter_Value"))
            names[key] = kn
        by_kernel = defaultdict(list)
        for key, cv in vals.items():
            by_kernel[names[key]].append(cv)
        for kn, ds in by_kernel.items():
            ndisp[kn] = max(ndisp[kn], len(ds))
            for c in ds[0]:
                merged[kn][c].append(statistics.mean(d.get(c, 0.0) for d in ds))
    out = [f"# Hardware counters{': ' + args.title if args.title else ''}", ""]
    if args.workload:
        out += [f"Workload: {args.workload}", ""]
    if args.cmd:
        out += ["Commands (from /tmp, repository at `$R`):", "", "```", *args.cmd, "```", ""]
    for kn, cs in merged.items():
        mean = {c: statistics.mean(v) for c, v in sorted(cs.items())}
        out += [f"`{kn[:120]}`: {ndisp[kn]} dispatches per pass, mean per dispatch:", "", "| counter | value |",
                "|---|---|"]
        for c, v in mean.items():
            out.append(f"| {c} | {v:.6g} |")
        out.append("")
        der = derived(mean)
        if der:
            out += ["Derived (256 CUs with one TA and one TD each, 1024 SIMDs; GRBM_GUI_ACTIVE is summed over "
                    "the 8 XCDs):", ""]
            out += [f"- {k}: {v}" for k, v in der]
            out.append("")
    if args.source_sha:
        out.append(f"kernel_source_sha: {args.source_sha}")
    print("\n".join(out))


def derived(m):
    """Shares and ratios from the raw counter means that are present."""
    d = []
    gui = m.get("GRBM_GUI_ACTIVE")
    per_xcd = gui / 8 if gui else None
    if per_xcd:
        for c, name in (("TA_TA_BUSY_sum", "TA busy share per CU"), ("TD_TD_BUSY_sum", "TD busy share per CU")):
            if c in m:
                d.append((name, f"{100 * m[c] / 256 / per_xcd:.1f} %"))
        if "SQ_VALU_MFMA_BUSY_CYCLES" in m:
            d.append(("MFMA busy share per SIMD", f"{100 * m['SQ_VALU_MFMA_BUSY_CYCLES'] / (per_xcd * 1024):.2f} %"))
        if "SQ_INSTS_VALU" in m:
            d.append(("VALU issue share per SIMD (4 cycles per wave64 instruction)",
                      f"{100 * 4 * m['SQ_INSTS_VALU'] / (per_xcd * 1024):.1f} %"))
    if "TCC_HIT_sum" in m and "TCC_MISS_sum" in m and m["TCC_HIT_sum"] + m["TCC_MISS_sum"] > 0:
        d.append(("L2 hit rate", f"{100 * m['TCC_HIT_sum'] / (m['TCC_HIT_sum'] + m['TCC_MISS_sum']):.1f} %"))
    if "SQ_LDS_BANK_CONFLICT" in m and "SQ_LDS_IDX_ACTIVE" in m and m["SQ_LDS_IDX_ACTIVE"] > m["SQ_LDS_BANK_CONFLICT"]:
        d.append(("LDS bank conflict ratio (conflict cycles / conflict-free active cycles)",
                  f"{m['SQ_LDS_BANK_CONFLICT'] / (m['SQ_LDS_IDX_ACTIVE'] - m['SQ_LDS_BANK_CONFLICT']):.3f}"))
    if "SQ_WAIT_INST_ANY" in m and m.get("SQ_WAVE_CYCLES"):
        d.append(("share of wave time waiting on memory", f"{100 * m['SQ_WAIT_INST_ANY'] / m['SQ_WAVE_CYCLES']:.1f} %"))
    if "SQ_INSTS_VALU_MFMA_MOPS_F16" in m:
        d.append(("MFMA work per dispatch", f"{m['SQ_INSTS_VALU_MFMA_MOPS_F16'] * 512 / 1e9:.1f} GFLOP"))
    return d


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    for name in ("router", "ceilings", "trace", "counters"):
        p = sub.add_parser(name)
        p.add_argument("file", nargs="+" if name == "counters" else None)
        p.add_argument("--cmd", action="append", default=[])
        if name == "trace":
            p.add_argument("--top", type=int, default=30)
        if name == "router":
            p.add_argument("--top", type=int, default=3)
            p.add_argument("--detail-below", type=float, default=0.99)
        if name == "counters":
            p.add_argument("--kernel", action="append", required=True)
            p.add_argument("--title", default="")
            p.add_argument("--workload", default="")
            p.add_argument("--source-sha", default="")
    p = sub.add_parser("traffic")
    p.add_argument("--fetch", required=True)
    p.add_argument("--write", required=True)
    p.add_argument("--kernel", action="append", required=True)
    p.add_argument("--algorithmic", required=True)
    p.add_argument("--workload", required=True)
    p.add_argument("--source-sha", required=True)
    p.add_argument("--cmd", action="append", default=[])
    args = ap.parse_args()
    {"router": router, "ceilings": ceilings, "trace": trace, "traffic": traffic, "counters": counters}[args.what](args)


if __name__ == "__main__":
    main()

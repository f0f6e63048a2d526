"""Benchmark of the CSR SpMM hot path on one MI355X.

One step = one spmm_run (all kernels of the product: light rows, split
pieces and their combine when the plan has them) over the headline workload:
the road-like graph (M = K = 1,000,000, Poisson(3) degrees, neighbours within
+-256 rows, unweighted) times B [1M, 64] fp32, sum reduction.  Inputs and the
plan are resident in HBM before timing starts.

Prints ONE JSON line on stdout (rank 0).  `value` is GFLOP/s = 2*nnz*N / t over
the K timed back-to-back steps.  Alongside: effective HBM GB/s on the
compulsory-byte model, the row kernel's roofline (achieved GB/s from HIP events
on the launch stream, against the 8 TB/s HBM peak), the CPU oracle timed on
this host, and per-regime results for the other synthetic graphs (warm
back-to-back and cache-flushed medians).

Byte model (compulsory bytes, per product): rowptr (M+1)*4 + nnz*(4 + 4 if
weighted) + K*N*4 (B) + M*N*4 (C) [+ M*N*8 argmax for max]; the plan stores
int32 indexes, so 4 bytes per index are what the kernels read.  Gather bytes
nnz*N*4 are reported beside it.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SpMM GFLOP/s (2·nnz·N) + effective HBM GB/s as % of MI355X peak, per regime"
HBM_PEAK_GBPS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["gnn_sparse_dense_amd/csrc/row_kernel_impl.h", "gnn_sparse_dense_amd/csrc/kernels.h"]
MFMA_SOURCES = ["gnn_sparse_dense_amd/csrc/mfma_tile.hip", "gnn_sparse_dense_amd/csrc/mfma_args.h"]
FAMILY_SOURCES = {"mfma_tile_kernel": MFMA_SOURCES, "mfma_split_tile_kernel": MFMA_SOURCES,
                  "split_fused_kernel": ["gnn_sparse_dense_amd/csrc/split_fused.hip"]}

REGIME_TEXT = {
    "tiny": "tiny random graph M=K=2,000, Poisson(8) degrees, 1% empty rows, weighted, N=16",
    "road": "road-like M=K=1,000,000, Poisson(3) degrees, neighbours within +-256 rows, unweighted, N=64",
    "powerlaw": "power-law M=K=2,000,000, degree exponent 2.1 rescaled to mean 25, max 50,000, "
                "uniform columns, GCN weights, N=128",
    "diffusion": "diffusion M=K=1,000,000, exactly 10 neighbours (Gaussian offsets sigma 500), "
                 "unweighted, N=16",
    "community": "community M=K=500,000 in 256-node blocks, Bernoulli(0.1) inside + 2 outside, "
                 "weighted, N=512",
    "mixed": "mixed M=K=1,000,000: a third road-like band, a third 256-node communities, a third "
             "power-law rows over all columns, weighted, N=128",
    "knn": "kNN line M=K=1,000,000, k=10 nearest points on a line, unweighted, N=64",
}


def kernel_source_hash(family: str = "") -> str:
    """Hash of the sources that define a kernel family's device code."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES + FAMILY_SOURCES.get(family, []):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def byte_model(g, N, reduce):
    idx = 4
    comp = (g.M + 1) * idx + g.nnz * (idx + (4 if g.val is not None else 0)) + g.K * N * 4 + g.M * N * 4
    if reduce == "max":
        comp += g.M * N * 8
    return comp, g.nnz * N * 4


def kernel_family(info) -> str:
    if info.get("route_mfma"):
        return "mfma_split_tile_kernel" if info.get("mfma_tiles") == 2 else "mfma_tile_kernel"
    if info.get("route_window"):
        return "window_sorted_kernel" if info.get("route_window") == 2 else "window_kernel"
    if info.get("route_tiled"):
        return "tile_kernel"
    if info.get("route_fused_split"):
        return "split_fused_kernel"
    return "row_kernel"


def read_traffic(family: str, workload: str):
    """Measured HBM bytes per launch from a committed rocprofv3 counter summary,
    or None when absent or taken on different kernel sources."""
    path = os.path.join(PROFILES, f"{family}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha") != kernel_source_hash(family):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class Runner:
    def set_width(self, N):
        """Swap in B [K, N] (the regime's feature recipe) and C [M, N]."""
        import workloads as W
        torch = self.torch
        if N == self.w.N:
            return
        dev = self.C.device
        self.B = self.C = self.arg = None
        torch.cuda.empty_cache()
        Bh = W.make_features(self.name, self.g.K, N)
        self.w = W.Workload(graph=self.g, N=N, B=Bh, reduces=self.w.reduces)
        self.B = torch.from_numpy(Bh).to(dev)
        self.C = torch.empty((self.g.M, N), dtype=torch.float32, device=dev)

    def __init__(self, name, M=None):
        import torch

        import gnn_sparse_dense_amd as G
        import workloads as W
        self.torch, self.G = torch, G
        self.name = name
        t0 = time.time()
        self.w = W.make(name, M=M)
        self.gen_s = time.time() - t0
        g = self.w.graph
        self.g = g
        dev = torch.device("cuda:0")
        self.rowptr = torch.from_numpy(g.rowptr).to(dev)
        self.col = torch.from_numpy(g.col).to(dev)
        self.val = None if g.val is None else torch.from_numpy(g.val).to(dev)
        self.B = torch.from_numpy(self.w.B).to(dev)
        self.C = torch.empty((g.M, self.w.N), dtype=torch.float32, device=dev)
        self.arg = None
        t0 = time.time()
        self.plan = G.spmm_plan_create(self.rowptr, self.col, self.val, g.M, g.K)
        self.plan_s = time.time() - t0
        self.info = G.spmm_plan_info(self.plan)

    def step(self, reduce):
        if reduce == "max" and self.arg is None:
            self.arg = self.torch.empty((self.g.M, self.w.N), dtype=self.torch.int64, device=self.C.device)
        self.G.spmm_run(self.plan, self.B, self.C, self.arg if reduce == "max" else None,
                        self.w.N, reduce, None)

    def time_steps(self, reduce, steps, warmup, flush=None):
        """Per-step durations (ms) from HIP events on the launch stream, plus the
        wall time of the whole back-to-back loop (ms) when flush is None."""
        torch = self.torch
        for _ in range(warmup):
            self.step(reduce)
        torch.cuda.synchronize()
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            if flush is not None:
                flush()
            starts[i].record()
            self.step(reduce)
            ends[i].record()
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t0) * 1e3
        return [s.elapsed_time(e) for s, e in zip(starts, ends)], wall_ms

    def time_back_to_back(self, reduce, steps, warmup):
        """K back-to-back steps with nothing recorded between them: one HIP
        event pair on the launch stream around the whole loop, the loop
        bracketed by synchronize on both sides.  Returns (GPU ms per step from
        the events, wall ms per step).  Events recorded between steps insert
        barrier packets that lengthen each step (road: 0.117 vs 0.109 ms)."""
        torch = self.torch
        for _ in range(warmup):
            self.step(reduce)
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        start.record()
        for _ in range(steps):
            self.step(reduce)
        end.record()
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t0) * 1e3
        return start.elapsed_time(end) / steps, wall_ms / steps

    def close(self):
        self.G.spmm_plan_destroy(self.plan)


def library_load_ms() -> float:
    import torch
    import gnn_sparse_dense_amd as G
    dev = torch.device("cuda:0")
    rp = torch.tensor([0, 1, 2], dtype=torch.int64, device=dev)
    cl = torch.tensor([1, 0], dtype=torch.int64, device=dev)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    G.spmm_plan_destroy(G.spmm_plan_create(rp, cl, None, 2, 2))
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3


def make_flush():
    import torch
    buf = torch.ones(512 * 1024 * 1024 // 4 * 2, dtype=torch.float32, device="cuda:0")   # 1 GiB

    def flush():
        buf.sum()          # reads 1 GiB: evicts L2 and the 256 MB Infinity Cache
    return flush


def copy_ceiling_gbps(reps=20):
    """Bandwidth of a plain 1 GiB device-to-device copy (bytes read + written)."""
    import torch
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    times = []
    for _ in range(reps):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        dst.copy_(src)
        e.record()
        e.synchronize()
        times.append(s.elapsed_time(e))
    del src, dst
    torch.cuda.empty_cache()
    return 2 * (1 << 30) / (statistics.median(times) * 1e-3) / 1e9


def _median_event_ms(fn, reps, flush=None):
    import torch
    times = []
    for _ in range(reps):
        if flush is not None:
            flush()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        e.synchronize()
        times.append(s.elapsed_time(e))
    return statistics.median(times)


def ceilings(flush, reps=20, gather_rows=500_000, gather_deg=16, N=128):
    """Bandwidth ceilings of this GPU, for reading the roofline fractions:
    * stream read, write and copy of 1 GiB with PyTorch's own kernels
      (sum, fill_, copy_), bytes moved / median event time;
    * the random-gather rate of the row kernel against the size of B: a graph
      of gather_rows rows with gather_deg uniform columns each over K rows of
      B [K, N=128] (512-byte rows), sum, 16 lanes per row in 64-column
      slices, for B from 32 MB to 1 GiB; gather bytes nnz * N * 4 / median
      time, warm (back to back) and with the caches flushed before each run."""
    import torch

    import gnn_sparse_dense_amd as G
    dev = torch.device("cuda:0")
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        src.sum()
        dst.fill_(1.0)
        dst.copy_(src)
    torch.cuda.synchronize()
    gib = n * 4
    rows2d = src.view(-1, 4096)
    readers = {"sum": lambda: src.sum(), "amax": lambda: src.amax(), "row sums [65536, 4096]": lambda: rows2d.sum(1),
               "count_nonzero": lambda: torch.count_nonzero(src)}
    read = {k: round(gib / (_median_event_ms(f, reps) * 1e-3) / 1e9, 1) for k, f in readers.items()}
    best = max(read, key=read.get)
    out = {"stream": {
        "read_GBps": read[best], "read_by_op": read,
        "write_GBps": round(gib / (_median_event_ms(lambda: dst.fill_(2.0), reps) * 1e-3) / 1e9, 1),
        "copy_GBps": round(2 * gib / (_median_event_ms(lambda: dst.copy_(src), reps) * 1e-3) / 1e9, 1),
        "bytes": gib, "kernels": f"torch {best} (fastest of {', '.join(read)}) / fill_ / copy_ over 1 GiB fp32",
        "reps": reps}}
    del src, dst
    torch.cuda.empty_cache()
    rows = [gather_rate(b_mb, flush, reps, gather_rows, gather_deg, N) for b_mb in (32, 64, 128, 256, 512, 1024)]
    out["gather"] = {"rows": gather_rows, "deg": gather_deg, "N": N, "gather_bytes": gather_rows * gather_deg * N * 4,
                     "by_B_size": rows}
    return out


def gather_rate(b_mb, flush, reps=20, M=500_000, gather_deg=16, N=128, lanes=16):
    """The row kernel's random-gather rate for B [K, N] of b_mb MB: M rows of
    gather_deg uniform columns, sum, `lanes` lanes per row (16: 64-column
    slices, the fastest mapping for uniform gathers from a large B, and the
    one skewed graphs are routed to; see ceilings())."""
    import torch

    import gnn_sparse_dense_amd as G
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(1234 + b_mb)
    nnz = M * gather_deg
    K = b_mb * (1 << 20) // (N * 4)
    rp = torch.arange(0, nnz + 1, gather_deg, dtype=torch.int64, device=dev)
    cl = torch.randint(0, K, (nnz,), dtype=torch.int64, device=dev, generator=gen)
    B = torch.randn((K, N), dtype=torch.float32, device=dev, generator=gen)
    C = torch.empty((M, N), dtype=torch.float32, device=dev)
    plan = G.spmm_plan_create(rp, cl, None, M, K)
    del rp, cl
    G.spmm_plan_set_option(plan, G.SPMM_OPT_LANES, lanes)

    def run():
        G.spmm_run(plan, B, C, None, N, "sum", None)
    for _ in range(5):
        run()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        run()
    e.record()
    e.synchronize()
    warm = s.elapsed_time(e) / reps
    cold = _median_event_ms(run, reps, flush)
    info = G.spmm_plan_info(plan)
    gbytes = nnz * N * 4
    row = {"B_MB": b_mb, "K": K, "warm_ms": round(warm, 5), "flushed_ms": round(cold, 5),
           "gather_GBps_warm": round(gbytes / (warm * 1e-3) / 1e9, 1),
           "gather_GBps_flushed": round(gbytes / (cold * 1e-3) / 1e9, 1),
           "route": [kernel_family(info), info["route_lanes"], info["route_vec"],
                     info["route_coarsen"], info["route_slices"]]}
    print(f"[bench] gather ceiling B={b_mb} MB: {row['gather_GBps_warm']} GB/s warm", file=sys.stderr,
          flush=True)
    G.spmm_plan_destroy(plan)
    del B, C
    torch.cuda.empty_cache()
    return row


def cpu_oracle_baseline(w, reduce, budget_s=10.0, max_reps=50):
    """The CPU oracle (single-threaded C, as built) on the headline workload:
    median time of repeated whole-graph runs, and the last run's output."""
    import oracle
    g = w.graph
    orc = oracle.default()
    times = []
    out = None
    t_start = time.perf_counter()
    while len(times) < max_reps:
        t0 = time.perf_counter()
        out = orc.spmm(g.rowptr, g.col, g.val, g.M, g.K, w.B, reduce)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start >= budget_s:
            break
    t = statistics.median(times)
    return t, len(times), out


def oracle_regime_timing(w, reduce, budget_elems=1e10, reps_small=3):
    """The single-threaded CPU oracle on one regime: the whole graph (median
    of reps_small runs when it is small, one run otherwise), or, past about
    budget_elems multiply-adds, one contiguous block of rows from the middle
    of the graph with its time scaled to the whole graph by entry count.
    Returns the timing record and the oracle's output (C, or (C, argmax) for
    max) with the rows it covers (None: all)."""
    import numpy as np

    import oracle
    g = w.graph
    orc = oracle.default()
    N = w.N
    total = g.nnz * N
    if total <= budget_elems:
        reps = reps_small if total <= 2e8 else 1
        rows, frac = None, 1.0
        what = f"the whole graph, median of {reps} runs" if reps > 1 else "the whole graph, one run"
    else:
        want = budget_elems / N                         # entries to cover
        deg = np.diff(g.rowptr)
        mid = g.M // 2
        cum = np.cumsum(deg[mid:])
        m = int(np.searchsorted(cum, want)) + 1
        rows = np.arange(mid, min(g.M, mid + m), dtype=np.int64)
        covered = int(g.rowptr[rows[-1] + 1] - g.rowptr[rows[0]])
        reps, frac = 1, covered / g.nnz
        what = f"rows {rows[0]}..{rows[-1]} ({covered} of {g.nnz} entries), one run, scaled by entry count"
    times = []
    out = None
    for _ in range(reps):
        t0 = time.perf_counter()
        out = orc.spmm(g.rowptr, g.col, g.val, g.M, g.K, w.B, reduce, rows=rows)
        times.append(time.perf_counter() - t0)
    t = statistics.median(times) / frac
    return ({"oracle_ms": round(t * 1e3, 2), "oracle_gflops": round(2.0 * total / t / 1e9, 3),
             "oracle_sample": what}, out, rows)


def parity_against_oracle(w, reduce, info, C, A, ref, rows=None):
    """The GPU output of the runs just timed against the oracle's output for
    the same inputs (the CPU-baseline leg's own run), on `rows` (None: all).
    Max: values and argmax bit for bit on every row.  Sum and mean: rows the
    row, tile and window kernels walk whole must equal the oracle's fused
    multiply-add mode bit for bit (same order, one rounding per entry); rows
    cut into pieces, and every row of the merge-path and panel routes, must
    lie within 1e-5 * sum|a*b| + 1e-6 (the sum of magnitudes from the oracle,
    in double, on those rows only)."""
    import numpy as np

    import oracle
    g = w.graph
    orc = oracle.default()
    sel = np.arange(g.M, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    Cg = C[sel] if rows is not None else C
    rec = {"rows_checked": int(sel.size), "outputs_checked": int(sel.size * w.N)}
    if reduce == "max":
        refC, refA = ref
        bad_v = int((Cg.view(np.uint32) != refC.view(np.uint32)).sum())
        Ag = A[sel] if rows is not None else A
        bad_a = int((Ag != refA).sum())
        rec.update({"rule": "bit-exact values and argmax", "value_mismatches": bad_v, "argmax_mismatches": bad_a,
                    "status": "ok" if bad_v == 0 and bad_a == 0 else "FAIL"})
        return rec
    deg = np.diff(g.rowptr)[sel]
    pieces = info["route_split"] and info["n_seg"] > 0
    loose_route = bool(info["route_merge"] or info["route_pairs"] or info["route_mfma"])
    whole = np.ones(sel.size, bool) if not pieces else deg <= info["split_T"]
    if loose_route:
        whole[:] = False
    fused = ref if g.val is None else orc.spmm(g.rowptr, g.col, g.val, g.M, g.K, w.B, reduce, fused=True,
                                                rows=rows)
    wi = np.flatnonzero(whole)
    bad_exact = int((Cg[wi].view(np.uint32) != fused[wi].view(np.uint32)).sum())
    li = np.flatnonzero(~whole)
    worst = 0.0
    bad_tol = 0
    if li.size:
        S = orc.sumabs(g.rowptr, g.col, g.val, g.M, w.B, rows=sel[li])
        err = np.abs(Cg[li].astype(np.float64) - ref[li].astype(np.float64))
        bound = 1e-5 * S + 1e-6
        bad_tol = int((~(err <= bound)).sum())
        worst = float(np.max(err / bound)) if err.size else 0.0
    rec.update({"rule": "whole rows bit-exact vs the fused oracle; other rows within 1e-5*sum|a*b| + 1e-6",
                "rows_bit_exact": int(wi.size), "rows_by_tolerance": int(li.size),
                "bit_mismatches": bad_exact, "tolerance_failures": bad_tol,
                "worst_err_over_bound": round(worst, 4),
                "status": "ok" if bad_exact == 0 and bad_tol == 0 else "FAIL"})
    return rec


def host_cpu() -> str:
    """The host's CPU model name and hardware thread count."""
    model = "unknown CPU"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return f"{model}, {os.cpu_count()} hardware threads"


def percentile(xs, q):
    xs = sorted(xs)
    return xs[min(len(xs) - 1, int(round(q * (len(xs) - 1))))]


def regime_result(r, reduce, steps, warmup, flush, cpu=False, gather_ceiling=None):
    g, N = r.g, r.w.N
    warm_ms, _ = r.time_back_to_back(reduce, steps, warmup)
    cold, _ = r.time_steps(reduce, steps, 2, flush=flush)
    r.info = r.G.spmm_plan_info(r.plan)       # routing of the runs just timed
    comp, gather = byte_model(g, N, reduce)
    med_c = statistics.median(cold)
    res = {
        "reduce": reduce, "M": g.M, "nnz": g.nnz, "N": N,
        "ms_flushed_median": round(med_c, 5), "ms_flushed_min": round(min(cold), 5),
        "ms_flushed_p90": round(percentile(cold, 0.9), 5),
        "ms_warm_back_to_back": round(warm_ms, 5),
        "gflops_flushed": round(2.0 * g.nnz * N / (med_c * 1e-3) / 1e9, 1),
        "effective_GBps_flushed": round(comp / (med_c * 1e-3) / 1e9, 1),
        "frac_hbm_peak_flushed": round(comp / (med_c * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "gather_GBps_flushed": round(gather / (med_c * 1e-3) / 1e9, 1),
        "compulsory_MB": round(comp / 1e6, 1), "gather_MB": round(gather / 1e6, 1),
        "path": kernel_family(r.info),
        "route": {k: r.info[k] for k in ("route_lanes", "route_vec", "route_coarsen",
                                         "route_rows_per_wave", "route_slices")},
        "split": {"T": r.info["split_T"], "L": r.info["split_L"], "n_heavy": r.info["n_heavy"],
                  "n_seg": r.info["n_seg"]},
        "plan_ms": round(r.info["plan_ms"], 2),
    }
    if gather_ceiling is not None:
        # gather-bound regimes: the gathered bytes against the random-gather
        # rate measured for a B of the same size
        achieved = gather / (med_c * 1e-3) / 1e9
        res["roofline_gather"] = {"bound": "gather", "achieved": round(achieved, 1),
                                  "peak": gather_ceiling["gather_GBps_flushed"], "unit": "GB/s",
                                  "frac": round(achieved / gather_ceiling["gather_GBps_flushed"], 4),
                                  "ceiling": f"random 512-byte gathers of the row kernel from a "
                                             f"{gather_ceiling['B_MB']} MB B, caches flushed"}
    if cpu:
        C = r.C.cpu().numpy()
        A = r.arg.cpu().numpy() if reduce == "max" else None
        o, ref, rows = oracle_regime_timing(r.w, reduce)
        o["gpu_speedup_vs_oracle"] = round(o["oracle_ms"] / med_c, 1)
        res.update(o)
        res["parity"] = parity_against_oracle(r.w, reduce, r.info, C, A, ref, rows)
        del C, A, ref
    return res


def tile_results(r, steps, warmup, flush, fp32_results=()):
    """The same regime on the matrix-core community tiles, for graphs the
    router sends to the community window kernel: fp16 tiles (their own looser
    contract) and split fp16 tiles (the fp32 contract), each with its build
    time and the runs that repay it against the fp32 route."""
    out = []
    for mode, contract in ((1, "fp16 tiles: 2e-3 * sum|a*b| + 1e-4"), (2, "split fp16 tiles: fp32 tolerance")):
        t0 = time.perf_counter()
        r.G.spmm_plan_set_option(r.plan, r.G.SPMM_OPT_MFMA, mode)
        build_ms = (time.perf_counter() - t0) * 1e3
        for red in r.w.reduces:
            if red == "max":
                continue
            res = regime_result(r, red, steps, warmup, flush)
            res["contract"] = contract
            res["tile_build_ms"] = round(build_ms, 2)
            fp32 = [x for x in fp32_results if x["reduce"] == red]
            if fp32:
                saving = fp32[0]["ms_flushed_median"] - res["ms_flushed_median"]
                res["break_even_runs"] = round(build_ms / saving, 1) if saving > 0 else None
            res["mfma_resid_nnz"] = r.info["mfma_resid_nnz"]
            out.append(res)
    r.G.spmm_plan_set_option(r.plan, r.G.SPMM_OPT_MFMA, 0)
    r.info = r.G.spmm_plan_info(r.plan)
    return out


def graph_replay_result(r, reduce, reps=100, rounds=20):
    """Launch-bound products captured in one HIP graph (reps products per graph)
    and replayed: microseconds per product, against eager back-to-back launches."""
    import torch
    G = r.G
    N = r.w.N
    arg = torch.empty((r.g.M, N), dtype=torch.int64, device=r.C.device) if reduce == "max" else None
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side, capture_error_mode="thread_local"):
        for _ in range(reps):
            G.spmm_run(r.plan, r.B, r.C, arg, N, reduce, None)
    graph.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(rounds):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        graph.replay()
        e.record()
        e.synchronize()
        times.append(s.elapsed_time(e) * 1e3 / reps)
    eager, wall_ms = r.time_steps(reduce, reps, 5)
    del graph
    return {"reduce": reduce, "us_per_product_graph": round(statistics.median(times), 2),
            "us_per_product_eager_wall": round(wall_ms * 1e3 / reps, 2),
            "us_per_launch_eager_events": round(statistics.median(eager) * 1e3, 2), "products_per_graph": reps}


def reuse_result(r, reduce, steps, flush):
    """First call against steady state (RA-SpMM, "When does RA-SpMM help?": a
    structure built once pays off after build / saving runs).  For each
    optional structure the router uses on this graph: its build time, the
    flushed per-run time with and without it, and the break-even run count."""
    G = r.G
    t_with = statistics.median(r.time_steps(reduce, steps, 2, flush=flush)[0])
    out = {"reduce": reduce, "plan_create_ms": round(r.info["plan_ms"], 3), "run_ms": round(t_with, 5),
           "first_call_ms": round(r.info["plan_ms"] + t_with, 3)}

    def structure(opt, off, auto):
        G.spmm_plan_set_option(r.plan, opt, off)
        t_off = statistics.median(r.time_steps(reduce, steps, 2, flush=flush)[0])
        t0 = time.perf_counter()
        G.spmm_plan_set_option(r.plan, opt, auto)
        build = (time.perf_counter() - t0) * 1e3
        saving = t_off - t_with
        return {"build_ms": round(build, 3), "ms_without": round(t_off, 5), "ms_with": round(t_with, 5),
                "break_even_runs": round(build / saving, 1) if saving > 0 else None}

    info = G.spmm_plan_info(r.plan)
    if info["route_tiled"]:
        out["row_tiles"] = structure(G.SPMM_OPT_TILES, 0, -1)
    if info["route_split"]:
        out["row_split"] = structure(G.SPMM_OPT_SPLIT_MODE, 0, -1)
    t0 = time.perf_counter()
    feat = G.spmm_plan_features(r.plan, 2)
    out["features_ms"] = round((time.perf_counter() - t0) * 1e3, 3)
    out["padding_ratio_V2"] = round(feat["padding_ratio"], 4)
    out["mean_row_bandwidth"] = round(feat["mean_bandwidth"], 1)
    r.info = G.spmm_plan_info(r.plan)
    return out


def vblock_result(steps, flush):
    """Vectorized blocking V = 2 (ParamSpMM section 3.1) where it is meant to
    pay: a k-nearest-neighbour graph of points on a line (M = K = 1,000,000,
    k = 10, unweighted, B [1M, 64]), row kernels against two-row panels."""
    import torch
    import gnn_sparse_dense_amd as G
    import workloads as W
    g = W.knn_line(1_000_000, 10)
    N = 64
    dev = torch.device("cuda:0")
    rp, cl = torch.from_numpy(g.rowptr).to(dev), torch.from_numpy(g.col).to(dev)
    B = torch.from_numpy(W.make_features("road", g.K, N)).to(dev)
    C = torch.empty((g.M, N), dtype=torch.float32, device=dev)
    plan = G.spmm_plan_create(rp, cl, None, g.M, g.K)
    auto_built = G.spmm_plan_info(plan)["pairs_built"]
    G.spmm_plan_set_option(plan, G.SPMM_OPT_VBLOCK, 0)          # the row kernels

    def run():
        G.spmm_run(plan, B, C, None, N, "sum", None)
    t_rows = time_flushed(run, flush, steps)
    t0 = time.perf_counter()
    G.spmm_plan_set_option(plan, G.SPMM_OPT_VBLOCK, -1)         # automatic: count, then build
    build = (time.perf_counter() - t0) * 1e3
    t_pan = time_flushed(run, flush, steps)
    info = G.spmm_plan_info(plan)
    G.spmm_plan_destroy(plan)
    comp, _ = byte_model(g, N, "sum")
    return {"workload": "kNN line M=K=1,000,000, k=10, unweighted, N=64, sum", "nnz": g.nnz,
            "padding_ratio": round(info["pair_padding"], 4), "routed_to_panels": info["route_pairs"],
            "built_at_plan_creation": auto_built,
            "ms_rows": round(t_rows, 5), "ms_panels": round(t_pan, 5), "speedup": round(t_rows / t_pan, 3),
            "effective_GBps_panels": round(comp / (t_pan * 1e-3) / 1e9, 1),
            "build_ms": round(build, 2),
            "break_even_runs": round(build / (t_rows - t_pan), 1) if t_rows > t_pan else None}


def reorder_result(steps, flush):
    """Locality reordering (reverse Cuthill-McKee, then P A P^T) on the road
    graph under random node ids: the kernels' time before and after, the
    one-time cost, and the runs that repay it."""
    import torch
    import gnn_sparse_dense_amd as G
    import workloads as W
    g = W.relabel(W.make_graph("road"), 74)
    N = 64
    dev = torch.device("cuda:0")
    rp, cl = torch.from_numpy(g.rowptr).to(dev), torch.from_numpy(g.col).to(dev)
    B = torch.from_numpy(W.make_features("road", g.K, N)).to(dev)
    C = torch.empty((g.M, N), dtype=torch.float32, device=dev)
    plan = G.spmm_plan_create(rp, cl, None, g.M, g.K)
    t_before = time_flushed(lambda: G.spmm_run(plan, B, C, None, N, "sum", None), flush, steps)
    # the first call in a process also loads the reordering kernels and the
    # library sorts; a second call on the same graph shows the steady cost
    t_rcm = []
    for _ in range(2):
        t0 = time.perf_counter()
        perm = G.spmm_plan_reorder(plan)
        torch.cuda.synchronize()
        t_rcm.append((time.perf_counter() - t0) * 1e3)
    t0 = time.perf_counter()
    pp = G.spmm_plan_permute(plan, perm)
    t_perm = (time.perf_counter() - t0) * 1e3
    Bp = B[perm].contiguous()
    t_after = time_flushed(lambda: G.spmm_run(pp, Bp, C, None, N, "sum", None), flush, steps)
    G.spmm_plan_destroy(pp)
    G.spmm_plan_destroy(plan)
    gain = t_before - t_after
    return {"workload": "road-like graph under random node ids (M=K=1,000,000, N=64, sum)",
            "ms_before": round(t_before, 5), "ms_after": round(t_after, 5),
            "speedup": round(t_before / t_after, 3), "rcm_first_call_ms": round(t_rcm[0], 1),
            "rcm_ms": round(t_rcm[1], 1), "permute_ms": round(t_perm, 1),
            "break_even_runs": round((t_rcm[1] + t_perm) / gain) if gain > 0 else None,
            "break_even_runs_first_call": round((t_rcm[0] + t_perm) / gain) if gain > 0 else None}


def router_sweep(r, reduce, steps, flush):
    """Router evidence (RA-SpMM abstract: the router's speed as a fraction of the
    best of all variants, per configuration): the router's choice against every
    forced (lanes, coarsening) pair and one-at-a-time toggles of its other
    decisions, all cache-flushed medians on one plan.  The fp16 tiles follow a
    looser contract and are listed apart, never counted as the best."""
    G = r.G
    auto = {G.SPMM_OPT_LANES: 0, G.SPMM_OPT_COARSEN: 0, G.SPMM_OPT_TILES: -1, G.SPMM_OPT_WINDOW: -1,
            G.SPMM_OPT_XCD_REMAP: -1, G.SPMM_OPT_NT_STORE: -1, G.SPMM_OPT_SPLIT_MODE: -1,
            G.SPMM_OPT_BALANCE: 0, G.SPMM_OPT_VBLOCK: -1, G.SPMM_OPT_SPLIT_FUSED: 1, G.SPMM_OPT_VEC: 0}
    variants = [("router", {})]
    variants += [(f"lanes={g} coarsen={f}", {G.SPMM_OPT_LANES: g, G.SPMM_OPT_COARSEN: f})
                 for g in (4, 8, 16, 32, 64) for f in (1, 2)]
    variants += [("row tiles off", {G.SPMM_OPT_TILES: 0}), ("row tiles compact", {G.SPMM_OPT_TILES: 1}),
                 ("row tiles wide", {G.SPMM_OPT_TILES: 2}), ("window on", {G.SPMM_OPT_WINDOW: 1}),
                 ("window off", {G.SPMM_OPT_WINDOW: 0}), ("XCD remap off", {G.SPMM_OPT_XCD_REMAP: 0}),
                 ("non-temporal C stores", {G.SPMM_OPT_NT_STORE: 1}), ("split on", {G.SPMM_OPT_SPLIT_MODE: 1}),
                 ("split off", {G.SPMM_OPT_SPLIT_MODE: 0}), ("merge-path balancing", {G.SPMM_OPT_BALANCE: 1}),
                 ("V = 2 panels", {G.SPMM_OPT_VBLOCK: 2}), ("V = 2 panels off", {G.SPMM_OPT_VBLOCK: 0}),
                 ("split in two dispatches", {G.SPMM_OPT_SPLIT_FUSED: 0}),
                 ("float2 lanes", {G.SPMM_OPT_VEC: 2}), ("float1 lanes", {G.SPMM_OPT_VEC: 1})]
    rows = []
    for label, opts in variants:
        print(f"[bench]   {reduce} {label}", file=sys.stderr, flush=True)
        entry = {"variant": label}
        try:
            for k, v in opts.items():
                G.spmm_plan_set_option(r.plan, k, v)
            ms = statistics.median(r.time_steps(reduce, steps, 2, flush=flush)[0])
            info = G.spmm_plan_info(r.plan)
            entry.update({"ms": round(ms, 5), "path": kernel_family(info) + ("+merge" if info["route_merge"] else "")
                          + ("+panels" if info["route_pairs"] else ""),
                          "route": [info["route_lanes"], info["route_vec"], info["route_coarsen"],
                                    info["route_slices"], info["route_xcd_remap"], info["route_nt_store"],
                                    info["route_split"], info["route_tiled"] * info["tiles"],
                                    info["route_window"]]})
        except G.SpmmError as e:
            entry["unsupported"] = str(e)
        finally:
            for k in opts:
                G.spmm_plan_set_option(r.plan, k, auto[k])
        rows.append(entry)
    timed = [x for x in rows if "ms" in x]
    # variants that resolve to the router's own kernel and launch shape time the
    # same code: the best of them is the router's figure, their spread the noise
    key = (rows[0]["path"], tuple(rows[0]["route"]))
    same = [x["ms"] for x in timed if (x["path"], tuple(x["route"])) == key]
    router_ms = min(same)
    best = min(timed, key=lambda x: x["ms"])
    out = {"reduce": reduce, "variants": rows, "router_ms": router_ms, "best_ms": best["ms"],
           "best_variant": best["variant"], "router_speed_vs_best": round(best["ms"] / router_ms, 4),
           "router_route_repeats": len(same),
           "router_route_spread": round(max(same) / min(same) - 1.0, 4)}
    if reduce != "max" and rows[0]["path"].startswith("window"):
        G.spmm_plan_set_option(r.plan, G.SPMM_OPT_MFMA, 1)
        ms = statistics.median(r.time_steps(reduce, steps, 2, flush=flush)[0])
        G.spmm_plan_set_option(r.plan, G.SPMM_OPT_MFMA, 0)
        out["fp16_tiles_ms"] = round(ms, 5)
    r.info = G.spmm_plan_info(r.plan)
    return out


def time_flushed(fn, flush, steps, warmup=3):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(steps):
        flush()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        e.synchronize()
        ts.append(s.elapsed_time(e))
    return statistics.median(ts)


def backward_result(r, flush, steps):
    """Backward pieces of one regime: the transposed plan (A^T, built once), the
    backward product dB = A^T dC of a sum, the max-pool backward where the
    regime reduces by max, and the stable edge-list -> CSR build."""
    import torch
    G, g, N = r.G, r.g, r.w.N
    dev = r.C.device
    # the process's first transpose also sets up the library sorts it uses:
    # the second build of the same transpose is the per-graph cost
    t_plans = []
    for _ in range(2):
        t0 = time.perf_counter()
        pt = G.spmm_plan_transpose(r.plan, 0)
        t_plans.append((time.perf_counter() - t0) * 1e3)
        if len(t_plans) == 1:
            G.spmm_plan_destroy(pt)
    t_plan = t_plans[1]
    dC = torch.randn((g.M, N), dtype=torch.float32, device=dev)
    dB = torch.empty((g.K, N), dtype=torch.float32, device=dev)
    ms = time_flushed(lambda: G.spmm_run(pt, dC, dB, None, N, "sum", None), flush, steps)
    comp_t = (g.K + 1) * 4 + g.nnz * (4 + (4 if g.val is not None else 0)) + g.M * N * 4 + g.K * N * 4
    out = {"transpose_plan_ms": round(t_plan, 2), "transpose_plan_first_ms": round(t_plans[0], 2),
           "sum_backward_ms": round(ms, 5),
           "sum_backward_GBps": round(comp_t / (ms * 1e-3) / 1e9, 1)}
    if "max" in r.w.reduces and g.val is None:
        arg = torch.empty((g.M, N), dtype=torch.int64, device=dev)
        G.spmm_run(r.plan, r.B, r.C, arg, N, "max", None)
        ms = time_flushed(lambda: G.spmm_max_backward(pt, arg, dC, dB, N, None), flush, steps)
        comp_m = (g.K + 1) * 4 + g.nnz * 4 + g.M * N * 12 + g.K * N * 4
        out.update({"max_backward_ms": round(ms, 5), "max_backward_GBps": round(comp_m / (ms * 1e-3) / 1e9, 1)})
    G.spmm_plan_destroy(pt)
    rows = torch.repeat_interleave(torch.arange(g.M, device=dev), torch.diff(r.rowptr))
    perm = torch.randperm(g.nnz, device=dev, generator=torch.Generator(device=dev).manual_seed(0))
    er, ec = rows[perm].contiguous(), r.col[perm].contiguous()
    ev = None if r.val is None else r.val[perm].contiguous()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    G.spmm_coo_to_csr(er, ec, ev, g.M, g.K)
    out["edge_list_to_csr_ms"] = round((time.perf_counter() - t0) * 1e3, 2)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="road", choices=sorted(REGIME_TEXT),
                    help="regime timed for the JSON line (default: the road-like headline)")
    ap.add_argument("--reduce", default=None, help="reduction for the JSON line (default: the regime's first)")
    ap.add_argument("--headline-only", action="store_true", help="skip the other regimes")
    ap.add_argument("--regimes", default="road,tiny,diffusion,community,powerlaw")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward timings")
    ap.add_argument("--mfma", type=int, nargs="?", const=1, default=0, choices=(0, 1, 2),
                    help="time the JSON-line workload on the matrix-core tiles: 1 fp16, 2 split fp16 (sum/mean)")
    ap.add_argument("--router-sweep", action="store_true",
                    help="only the router evidence: every forced variant per regime against the router's pick")
    ap.add_argument("--widths", default="",
                    help="router sweep: feature widths N to sweep per regime (default: each regime's own)")
    ap.add_argument("--ceilings", action="store_true",
                    help="only the bandwidth ceilings: stream read, write and copy of 1 GiB, and the row "
                         "kernel's random-gather rate against the size of B")
    ap.add_argument("--option", action="append", default=[], metavar="NAME=VALUE",
                    help="set a plan option on the JSON-line workload's plan, e.g. PIECE_ORDER=0 "
                         "(SPMM_OPT_<NAME>; repeatable)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(rows would shard with a per-layer halo exchange of B; see the design notes).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    if args.ceilings:
        print(json.dumps({"ceilings": ceilings(make_flush(), reps=min(args.steps, 20))}), flush=True)
        return

    if args.router_sweep:
        flush = make_flush()
        evidence = {}
        widths = [int(x) for x in args.widths.split(",") if x] if args.widths else []
        for name in [x for x in args.regimes.split(",") if x]:
            rr = Runner(name)
            base_N = rr.w.N
            for N in (widths or [base_N]):
                rr.set_width(N)
                reds = rr.w.reduces if N == base_N else rr.w.reduces[:1]
                print(f"[bench] router sweep {name}: M={rr.g.M} nnz={rr.g.nnz} N={N} {','.join(reds)}",
                      file=sys.stderr, flush=True)
                evidence[f"{name}/N={N}"] = [router_sweep(rr, red, min(args.steps, 30), flush) for red in reds]
            rr.close()
            del rr
            torch.cuda.empty_cache()
        ratios = [x["router_speed_vs_best"] for v in evidence.values() for x in v]
        geo = 1.0
        for q in ratios:
            geo *= q
        print(json.dumps({"router_evidence": evidence, "steps": min(args.steps, 30),
                          "router_speed_vs_best_geomean": round(geo ** (1.0 / len(ratios)), 4),
                          "router_speed_vs_best_min": min(ratios)}), flush=True)
        return

    # the process's first library call loads the library's code object onto
    # the GPU (about 13 ms); a throwaway plan on a 2-node graph pays it here,
    # so that each graph's plan creation below is its own cost
    load_ms = library_load_ms()
    headline = args.workload
    r = Runner(headline)
    reduce = args.reduce or r.w.reduces[0]
    g, N = r.g, r.w.N
    print(f"[bench] {headline}: M={g.M} nnz={g.nnz} N={N} gen={r.gen_s:.1f}s plan={r.info['plan_ms']:.1f}ms",
          file=sys.stderr, flush=True)
    if args.mfma:
        assert reduce != "max", "the fp16 tiles serve sum and mean only"
        r.G.spmm_plan_set_option(r.plan, r.G.SPMM_OPT_MFMA, args.mfma)
    for opt in args.option:
        name, _, value = opt.partition("=")
        r.G.spmm_plan_set_option(r.plan, getattr(r.G, "SPMM_OPT_" + name.strip().upper()), int(value))
        print(f"[bench] option SPMM_OPT_{name.strip().upper()} = {int(value)}", file=sys.stderr, flush=True)
    if args.option:
        r.info = r.G.spmm_plan_info(r.plan)
        result_options = {o.partition("=")[0].strip().upper(): int(o.partition("=")[2]) for o in args.option}
    else:
        result_options = None

    copy_gbps = copy_ceiling_gbps(reps=3 if args.calibrate_copy else 20)

    # one spmm_run per step; for this route it is one kernel launch, so the
    # event time per step is that kernel's average launch duration
    avg_launch_ms, ms_per_step = r.time_back_to_back(reduce, args.steps, args.warmup)
    r.info = r.G.spmm_plan_info(r.plan)       # routing of the runs just timed
    # kernel launches per product: the split adds a piece pass and a combine
    # per 256 columns, the merge path a fix-up; with more than one launch the
    # event time per step covers all of them
    launches = 2 if r.info["route_merge"] else 1
    if r.info["route_split"] and r.info["n_seg"] > 0:
        # one combine per pass; the pieces share the row kernel's dispatch
        # when the split runs fused, else add a launch per pass
        launches += (1 if r.info["route_fused_split"] else 2) * (-(-N // 256))
    comp, gather = byte_model(g, N, reduce)
    flops = 2.0 * g.nnz * N
    value = flops / (ms_per_step * 1e-3) / 1e9
    achieved = comp / (avg_launch_ms * 1e-3) / 1e9
    family = kernel_family(r.info)
    traffic = read_traffic(family, headline)

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {0: "f32", 1: "f16 tiles + f32", 2: "split f16 tiles + f32"}[args.mfma],
        "data": "synthetic",
        "config": {"workload": REGIME_TEXT[headline] + f", {reduce} reduction", "M": g.M, "K": g.K,
                   "nnz": g.nnz, "N": N, "reduce": reduce, "index_bits": 32,
                   **({"options": result_options} if result_options else {})},
        "effective_GBps": round(comp / (ms_per_step * 1e-3) / 1e9, 1),
        "frac_of_hbm_peak": round(comp / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "gather_GBps": round(gather / (ms_per_step * 1e-3) / 1e9, 1),
        "hbm_copy_ceiling_GBps": round(copy_gbps, 1),
        "frac_of_copy_ceiling": round(comp / (ms_per_step * 1e-3) / 1e9 / copy_gbps, 4),
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": None if traffic is None else round(traffic),
            "kernel": "%s_t (lanes=%d vec=%d coarsen=%d)" % (
                family, r.info["route_lanes"], r.info["route_vec"], r.info["route_coarsen"]),
            "bytes_per_launch": comp, "avg_launch_ms": round(avg_launch_ms, 5),
            "launches_per_step": launches,
            "timing": "warm: one HIP event pair on the launch stream around the K back-to-back timed steps "
                      "(synchronize on both sides), divided by K; caches not flushed",
        },
    }

    if not args.no_cpu:
        # the output of the last timed step, checked against the oracle run
        # that the CPU baseline times
        C_gpu = r.C.cpu().numpy()
        A_gpu = r.arg.cpu().numpy() if reduce == "max" else None
        t_cpu, reps, ref = cpu_oracle_baseline(r.w, reduce)
        result["cpu_baseline"] = {
            "value": round(flops / t_cpu / 1e9, 3), "unit": "GFLOP/s", "cores": 1, "kind": "oracle",
            "sample": f"the full {headline} graph and B, {reduce}, median of {reps} single-threaded "
                      f"oracle runs ({t_cpu * 1e3:.1f} ms each) on {host_cpu()}",
        }
        headline_parity = parity_against_oracle(r.w, reduce, r.info, C_gpu, A_gpu, ref)
        result["parity"] = headline_parity["status"]
        result["parity_detail"] = {"headline": headline_parity}
        del C_gpu, A_gpu, ref
        print(f"[bench] parity {headline} {reduce}: {headline_parity['status']}", file=sys.stderr, flush=True)

    if not args.headline_only:
        flush = make_flush()
        regimes, backward, reuse = {}, {}, {}
        regimes[headline] = [regime_result(r, red, args.steps, min(args.warmup, 50), flush, cpu=not args.no_cpu)
                             for red in r.w.reduces]
        if r.info["route_window"] and not args.mfma:
            regimes[headline] += tile_results(r, args.steps, min(args.warmup, 50), flush, regimes[headline])
        reuse[headline] = reuse_result(r, r.w.reduces[0], min(args.steps, 50), flush)
        if not args.no_backward:
            backward[headline] = backward_result(r, flush, min(args.steps, 50))
        r.close()
        del r
        torch.cuda.empty_cache()
        for name in [x for x in args.regimes.split(",") if x and x != headline]:
            rr = Runner(name)
            print(f"[bench] {name}: M={rr.g.M} nnz={rr.g.nnz} N={rr.w.N} gen={rr.gen_s:.1f}s",
                  file=sys.stderr, flush=True)
            gceil = None
            if name == "powerlaw":
                gceil = gather_rate(1024, flush, reps=min(args.steps, 20))
            regimes[name] = [regime_result(rr, red, args.steps, min(args.warmup, 50), flush, cpu=not args.no_cpu,
                                           gather_ceiling=gceil) for red in rr.w.reduces]
            if rr.info["route_window"]:
                regimes[name] += tile_results(rr, args.steps, min(args.warmup, 50), flush, regimes[name])
            reuse[name] = reuse_result(rr, rr.w.reduces[0], min(args.steps, 50), flush)
            if name == "tiny":
                reuse[name]["graph_replay"] = graph_replay_result(rr, rr.w.reduces[0])
            if not args.no_backward:
                backward[name] = backward_result(rr, flush, min(args.steps, 50))
            rr.close()
            del rr
            torch.cuda.empty_cache()
        result["regimes"] = regimes
        same = [x for x in regimes[headline] if x["reduce"] == reduce and "contract" not in x]
        if same:
            # the same launch with the caches flushed before each run (the
            # protocol the per-regime figures use), for comparison
            result["roofline"]["frac_flushed"] = same[0]["frac_hbm_peak_flushed"]
            result["roofline"]["avg_launch_ms_flushed"] = same[0]["ms_flushed_median"]
        if not args.no_cpu:
            checks = {f"{name}/{x['reduce']}": x["parity"]["status"] for name, xs in regimes.items() for x in xs
                      if "parity" in x}
            result["parity_detail"]["regimes"] = checks
            if any(v != "ok" for v in checks.values()):
                result["parity"] = "FAIL"
        result["reuse"] = dict(reuse, library_load_ms=round(load_ms, 2))
        result["vblock"] = vblock_result(min(args.steps, 50), flush)
        result["reorder"] = reorder_result(min(args.steps, 50), flush)
        if backward:
            result["backward"] = backward
    else:
        r.close()

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

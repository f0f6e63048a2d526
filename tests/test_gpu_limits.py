"""GPU parity at the library's index limits, through the C ABI.

A plan accepts M, K and nnz up to 2^31 - 2 (the device keeps int32 indexes).
Two graphs sit at those limits.  They are built on the device from the
integer formulas in ``workloads`` (hashed_cols, small_int_features,
alternating_rowptr, limit_degrees) and checked on sampled rows against the
oracle, which gets those rows rebuilt on the host from the same formulas
(columns renumbered densely in sorted order; the stored order is kept, so
sums, maxima and the tie order do not change):

* nnz = 2^31 - 2 over 4M rows: light rows of up to 700 entries, 63 rows of
  about 10M entries, and a last row of 2^25 entries whose last piece ends at
  the last entry position.  The row split's partition is compared in full.
  With the split switched off, the 10M-entry rows run whole (bit-exact
  against the oracle) and the 2^25-entry row is still split: no row of more
  than 2^24 entries is walked whole.
* M = K = 2^31 - 2 (odd rows hold one entry, even rows none), N = 1, with
  row tiles forced on and off.  Every one of the 2^31 - 2 outputs (and
  argmax) is also compared with the value the formulas give, exactly (B
  holds small integers), which covers every dispatch of the launch.
"""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gnn_sparse_dense_amd as G
    from tests.gpu_helpers import ABS_TOL, DEV, REL_TOL, log

LIMIT = 2**31 - 2
CHUNK = 1 << 27                  # elements per device-side generation step
MAX_WHOLE_ROW = 1 << 24          # longest row the kernels walk whole


def _arange(s, e):
    return torch.arange(s, e, dtype=torch.int64, device=DEV)


def _sub_problem(rows, starts, deg, colfn, bfn):
    """Rows `rows` (entries [starts, starts + deg)) as a small graph: columns
    renumbered to 0..u-1 in sorted order, B restricted to the u used rows.
    Returns (graph, B_sub, used columns)."""
    total = int(deg.sum())
    offs = np.zeros(rows.size + 1, np.int64)
    np.cumsum(deg, out=offs[1:])
    pos = np.repeat(starts - offs[:-1], deg) + np.arange(total, dtype=np.int64)
    cols = colfn(pos)
    used, local = np.unique(cols, return_inverse=True)
    g = W.Graph("sampled", rows.size, used.size, offs, local.astype(np.int64), None)
    return g, bfn(used), used


def _check_sampled(orc, g, Bs, used, red, C, arg, exact, what):
    """C, arg: GPU results of the sampled rows; exact: indexes (into the
    sample) of rows that ran whole, bit-exact against the oracle."""
    if red == "max":
        refC, refA = orc.spmm(g.rowptr, g.col, None, g.M, g.K, Bs, "max")
        assert np.array_equal(C.view(np.uint32), refC.view(np.uint32)), f"{what}: max values"
        refA = np.where(refA >= 0, used[np.maximum(refA, 0)], -1)
        assert np.array_equal(arg, refA), f"{what}: argmax"
        return
    ref = orc.spmm(g.rowptr, g.col, None, g.M, g.K, Bs, red)
    S = orc.sumabs(g.rowptr, g.col, None, g.M, Bs)
    err = np.abs(C.astype(np.float64) - ref.astype(np.float64))
    assert np.all(err <= REL_TOL * S + ABS_TOL), f"{what}: max err {err.max():.3e}"
    if len(exact):
        assert np.array_equal(C[exact].view(np.uint32), ref[exact].view(np.uint32)), f"{what}: whole rows"


def _run(plan, Bd, M, red):
    N = Bd.shape[1]
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    arg = torch.full((M, N), 0x7F7F7F7F, dtype=torch.int64, device=DEV) if red == "max" else None
    G.spmm_run(plan, Bd, C, arg, N, red)
    torch.cuda.synchronize()
    return C, arg


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_max_nnz(orc):
    M, K, N = 1 << 22, (1 << 24) + 3, 4
    deg = W.limit_degrees(M, LIMIT, 63, 1 << 25)
    rowptr = np.zeros(M + 1, np.int64)
    np.cumsum(deg, out=rowptr[1:])
    rng = np.random.default_rng(31)
    B = rng.standard_normal((K, N)).astype(np.float32)
    log(f"limits: nnz={LIMIT} M={M} K={K}: building the columns on the device")
    rp_d = torch.from_numpy(rowptr).to(DEV)
    col_d = torch.empty(LIMIT, dtype=torch.int64, device=DEV)
    for s in range(0, LIMIT, CHUNK):
        e = min(s + CHUNK, LIMIT)
        col_d[s:e] = W.hashed_cols(_arange(s, e), K)
    log("limits: plan")
    plan = G.spmm_plan_create(rp_d, col_d, None, M, K)
    del col_d, rp_d
    _free()
    info = G.spmm_plan_info(plan)
    assert info["nnz"] == LIMIT and info["dmax"] == 1 << 25
    T, L = info["split_T"], info["split_L"]
    assert info["n_heavy"] == 64 and T < 700 * 2 and L <= MAX_WHOLE_ROW
    part = G.spmm_plan_partition(plan)
    ref = orc.partition(rowptr, M, T, L)
    assert part["n_heavy"] == ref["n_heavy"] == 64
    for k in ("seg_row", "seg_begin", "seg_end", "light"):
        assert np.array_equal(part[k], ref[k]), k
    assert part["seg_end"][-1] == LIMIT

    heavy = np.flatnonzero(deg > T)
    sample = np.unique(np.concatenate([np.arange(32), np.arange(M - 32, M), heavy[[0, 31]],
                                       rng.choice(M, size=200, replace=False)])).astype(np.int64)
    g, Bs, used = _sub_problem(sample, rowptr[sample], deg[sample], lambda p: W.hashed_cols(p, K),
                               lambda u: B[u])
    Bd = torch.from_numpy(B).to(DEV)
    whole = np.flatnonzero(deg[sample] <= T)
    for red in ("sum", "mean", "max"):
        log(f"limits nnz: {red} N={N}")
        C, arg = _run(plan, Bd, M, red)
        Cs = C[torch.from_numpy(sample).to(DEV)].cpu().numpy()
        As = None if arg is None else arg[torch.from_numpy(sample).to(DEV)].cpu().numpy()
        del C, arg
        _check_sampled(orc, g, Bs, used, red, Cs, As, whole, f"nnz limit {red}")
    log("limits nnz: sum N=1")
    C, _ = _run(plan, Bd[:, :1].contiguous(), M, "sum")
    Cs = C[torch.from_numpy(sample).to(DEV)].cpu().numpy()
    del C
    _check_sampled(orc, g, np.ascontiguousarray(Bs[:, :1]), used, "sum", Cs, None, whole, "nnz limit N=1")

    # split off: only the row above 2^24 entries is still split
    G.spmm_plan_set_option(plan, G.SPMM_OPT_SPLIT_MODE, 0)
    info = G.spmm_plan_info(plan)
    assert info["split_T"] == MAX_WHOLE_ROW and info["n_heavy"] == 1
    part = G.spmm_plan_partition(plan)
    ref = orc.partition(rowptr, M, MAX_WHOLE_ROW, info["split_L"])
    for k in ("seg_row", "seg_begin", "seg_end", "light"):
        assert np.array_equal(part[k], ref[k]), f"split off: {k}"
    whole = np.flatnonzero(deg[sample] <= MAX_WHOLE_ROW)
    for red in ("sum", "max"):
        log(f"limits nnz, split off: {red}")
        C, arg = _run(plan, Bd, M, red)
        Cs = C[torch.from_numpy(sample).to(DEV)].cpu().numpy()
        As = None if arg is None else arg[torch.from_numpy(sample).to(DEV)].cpu().numpy()
        del C, arg
        _check_sampled(orc, g, Bs, used, red, Cs, As, whole, f"nnz limit split off {red}")
    G.spmm_plan_destroy(plan)
    del Bd
    _free()


def test_max_rows(orc):
    M = K = LIMIT
    nnz = int(W.alternating_rowptr(np.int64(M)))
    log(f"limits: M=K={M} nnz={nnz}: building rowptr and columns on the device")
    rp_d = torch.empty(M + 1, dtype=torch.int64, device=DEV)
    for s in range(0, M + 1, CHUNK):
        e = min(s + CHUNK, M + 1)
        rp_d[s:e] = W.alternating_rowptr(_arange(s, e))
    col_d = torch.empty(nnz, dtype=torch.int64, device=DEV)
    for s in range(0, nnz, CHUNK):
        e = min(s + CHUNK, nnz)
        col_d[s:e] = W.hashed_cols(_arange(s, e), K)
    log("limits rows: plan")
    plan = G.spmm_plan_create(rp_d, col_d, None, M, K)
    del rp_d, col_d
    _free()
    info = G.spmm_plan_info(plan)
    assert info["M"] == M and info["nnz"] == nnz and info["dmax"] == 1 and info["n_empty"] == M - nnz
    Bd = torch.empty((K, 1), dtype=torch.float32, device=DEV)
    for s in range(0, K, CHUNK):
        e = min(s + CHUNK, K)
        Bd[s:e, 0] = W.small_int_features(_arange(s, e)).to(torch.float32)

    rng = np.random.default_rng(37)
    sample = np.unique(np.concatenate([np.arange(64), np.arange(M - 64, M),
                                       rng.choice(M, size=2000, replace=False)])).astype(np.int64)
    starts = W.alternating_rowptr(sample)
    g, Bs, used = _sub_problem(sample, starts, W.alternating_rowptr(sample + 1) - starts,
                               lambda p: W.hashed_cols(p, K),
                               lambda u: W.small_int_features(u).astype(np.float32).reshape(-1, 1))
    sample_d = torch.from_numpy(sample).to(DEV)
    for tiles in (1, 0):
        G.spmm_plan_set_option(plan, G.SPMM_OPT_TILES, tiles)
        for red in (("sum", "mean", "max") if tiles else ("sum", "max")):
            log(f"limits rows: tiles={tiles} {red}")
            C, arg = _run(plan, Bd, M, red)
            assert G.spmm_plan_info(plan)["route_tiled"] == tiles
            # every output against the formulas (one entry per odd row: the sum,
            # mean and maximum are that entry's B value, argmax its column)
            for s in range(0, M, CHUNK):
                e = min(s + CHUNK, M)
                i = _arange(s, e)
                odd = (i % 2) == 1
                c = W.hashed_cols(W.alternating_rowptr(i), K)
                want = torch.where(odd, W.small_int_features(c).to(torch.float32), torch.zeros((), device=DEV))
                assert torch.equal(C[s:e, 0].view(torch.int32), want.view(torch.int32)), f"rows {s}..{e}"
                if arg is not None:
                    assert torch.equal(arg[s:e, 0], torch.where(odd, c, torch.full((), -1, device=DEV))), \
                        f"argmax rows {s}..{e}"
                del i, odd, c, want
            Cs = C[sample_d].cpu().numpy()
            As = None if arg is None else arg[sample_d].cpu().numpy()
            del C, arg
            _free()
            _check_sampled(orc, g, Bs, used, red, Cs, As, np.arange(sample.size), f"rows limit tiles={tiles} {red}")
    G.spmm_plan_destroy(plan)
    del Bd
    _free()

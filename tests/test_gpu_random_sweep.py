"""GPU parity over a seeded sweep of random graphs, widths, reductions and
plan options (every router decision forced on, off or left automatic, in
random combinations), through the C ABI, against the oracle: sum and mean
within the tolerance, max and argmax bit-exact, rows walked whole bit-exact
against the fused oracle.  B, C and argmax start one element past an
allocation's start in about half the cases (rows only 4- or 8-byte
aligned), and the elements next to C and argmax must stay untouched.
Combinations the library refuses as unsupported are counted, not failed."""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gnn_sparse_dense_amd as G
    from tests.gpu_helpers import DEV, check, gpu_run, log, make_plan, to_dev

CASES = 300


def _options(rng):
    pick = lambda xs: xs[int(rng.integers(len(xs)))]
    opts = []
    mode = pick([-1, 0, 1])
    opts.append((G.SPMM_OPT_SPLIT_MODE, mode))
    if mode == 1:
        opts += [(G.SPMM_OPT_SPLIT_T, int(rng.integers(16, 400))), (G.SPMM_OPT_SPLIT_L, int(rng.integers(8, 300)))]
    opts += [(G.SPMM_OPT_TILES, pick([-1, 0, 1, 2])), (G.SPMM_OPT_WINDOW, pick([-1, 0, 1])),
             (G.SPMM_OPT_VBLOCK, pick([-1, 0, 2])), (G.SPMM_OPT_BALANCE, pick([0, 0, 1])),
             (G.SPMM_OPT_SPLIT_FUSED, pick([0, 1])), (G.SPMM_OPT_PIECE_ORDER, pick([0, 1])),
             (G.SPMM_OPT_XCD_REMAP, pick([-1, 0, 1])), (G.SPMM_OPT_NT_STORE, pick([-1, 0, 1]))]
    if rng.random() < 0.5:
        opts += [(G.SPMM_OPT_LANES, pick([4, 8, 16, 32, 64])), (G.SPMM_OPT_COARSEN, pick([1, 2])),
                 (G.SPMM_OPT_VEC, pick([1, 2, 4]))]
    return opts


def _graph(rng):
    u = rng.random()
    if u < 0.15:   # communities of 256 nodes: the window kernels' graphs
        g = W.make_graph("community", M=int(rng.integers(300, 5000)))
        return W.relabel(g, int(rng.integers(1 << 30))) if rng.random() < 0.3 else g
    if u < 0.2:    # the power-law recipe (its hubs need M above the largest degree)
        return W.make_graph("powerlaw", M=int(rng.integers(60_000, 80_000)))
    M = int(rng.integers(1, 4000))
    K = int(rng.integers(1, 4000))
    heavy = int(rng.integers(0, 6))
    return W.random_csr(rng, M, K, mean_deg=float(rng.uniform(0.5, 30.0)), empty_frac=float(rng.uniform(0, 0.3)),
                        dup_frac=float(rng.uniform(0, 0.2)), shuffle_rows=bool(rng.random() < 0.5),
                        zero_frac=float(rng.uniform(0, 0.05)), weighted=bool(rng.random() < 0.6),
                        heavy_rows=heavy, heavy_deg=int(rng.integers(100, 3000)) if heavy else 0)


def test_random_sweep(orc):
    rng = np.random.default_rng(20261202)
    refused = 0
    routes = {}
    for case in range(CASES):
        g = _graph(rng)
        N = int(rng.choice([1, 3, 4, 5, 6, 7, 9, 13, 16, 17, 33, 50, 64, 66, 100, 130, 200, 257, 258, 259, 300, 513]))
        red = ["sum", "mean", "max"][int(rng.integers(3))]
        opts = _options(rng)
        what = f"case {case}: M={g.M} K={g.K} nnz={g.nnz} N={N} {red} opts={opts}"
        log(what)
        try:
            plan = make_plan(g, opts)
        except G.SpmmError as e:
            assert e.status == G.SPMM_E_UNSUPPORTED, f"{what}: {e}"
            refused += 1
            continue
        B = rng.standard_normal((g.K, N)).astype(np.float32)
        _, _, _, Bd0 = to_dev(g, B)
        ob, oc = int(rng.integers(2)), int(rng.integers(2))
        log(f"  offsets B {ob} C {oc}")
        Bbig = torch.empty(g.K * N + 1, dtype=torch.float32, device=DEV)
        Bd = Bbig[ob:ob + g.K * N].view(g.K, N)
        Bd.copy_(Bd0)
        try:
            Cbig = torch.full((g.M * N + 2,), float("nan"), dtype=torch.float32, device=DEV)
            Cv = Cbig[oc:oc + g.M * N].view(g.M, N)
            Abig = None
            Av = None
            if red == "max":
                Abig = torch.full((g.M * N + 2,), 0x7F7F7F7F7F7F7F7F, dtype=torch.int64, device=DEV)
                Av = Abig[oc:oc + g.M * N].view(g.M, N)
            G.spmm_run(plan, Bd, Cv, Av, N, red, None)
            torch.cuda.synchronize()
            C = Cv.cpu().numpy()
            arg = None if Av is None else Av.cpu().numpy()
            tail = Cbig[oc + g.M * N:].cpu().numpy()
            assert np.isnan(tail).all(), f"{what}: write past C"
            if oc:
                assert np.isnan(Cbig[0].item()), f"{what}: write before C"
            if Abig is not None:
                atail = Abig[oc + g.M * N:].cpu().numpy()
                assert (atail == 0x7F7F7F7F7F7F7F7F).all(), f"{what}: write past argmax"
        except G.SpmmError as e:
            assert e.status == G.SPMM_E_UNSUPPORTED, f"{what}: {e}"
            refused += 1
            G.spmm_plan_destroy(plan)
            continue
        info = G.spmm_plan_info(plan)
        key = ("merge" if info["route_merge"] else "panels" if info["route_pairs"] else
               "window" if info["route_window"] else "tiles" if info["route_tiled"] else "rows") + \
              ("+split" if info["route_split"] and info["n_seg"] > 0 else "") + \
              ("+one dispatch" if info["route_fused_split"] else "") + f"/v{info['route_vec']}"
        routes[key] = routes.get(key, 0) + 1
        # rows walked whole: all of them, less the split rows; none certified
        # on the merge path (a row may span segments) or on V = 2 panels over
        # rows not stored in column order (entries taken in panel order)
        exact = None
        if not info["route_merge"] and not (info["route_pairs"] and info["pairs_built"] == 2):
            exact = G.spmm_plan_partition(plan)["light"] if info["route_split"] and info["n_seg"] > 0 \
                else np.arange(g.M)
        check(orc, g, B, red, C, arg, exact_rows=exact, what=what)
        G.spmm_plan_destroy(plan)
    log(f"random sweep: {CASES - refused} cases run, {refused} refused as unsupported; routes {routes}")
    assert refused < CASES // 2

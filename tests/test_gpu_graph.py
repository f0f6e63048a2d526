"""spmm_run inside a captured HIP graph (the launch-bound case: capture once,
replay per layer).  The product path enqueues kernels only (no memset or
copy), so every route can be captured; each case is replayed several times
with unrelated eager work and synchronisations in between, and every replay
must reproduce the eager result bit for bit."""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gnn_sparse_dense_amd as G
    from tests.gpu_helpers import DEV, check, log, make_plan, to_dev

CASES = {
    "road-tiles": (lambda: W.make_graph("road", M=40_000), (), 64, "sum"),
    "powerlaw-split": (lambda: W.make_graph("powerlaw", M=60_000), (), 128, "sum"),
    "community-window": (lambda: W.make_graph("community", M=6_000), (), 512, "sum"),
    "tiny-max": (lambda: W.make_graph("tiny"), (), 16, "max"),
    "merge": (lambda: W.random_csr(np.random.default_rng(8), 5000, 4000, mean_deg=6.0, heavy_rows=4,
                                   heavy_deg=3000, shuffle_rows=True), "merge", 96, "mean"),
    "panels": (lambda: W.knn_line(20_000, 10), "panels", 32, "sum"),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_graph_capture_replay(orc, case):
    make, opts, N, red = CASES[case]
    g = make()
    options = {"merge": ((G.SPMM_OPT_BALANCE, 1),), "panels": ((G.SPMM_OPT_VBLOCK, 2),)}.get(opts, ())
    plan = make_plan(g, options)
    rng = np.random.default_rng(N)
    B = rng.standard_normal((g.K, N)).astype(np.float32)
    _, _, _, Bd = to_dev(g, B)
    is_max = red == "max"
    C_ref = torch.empty((g.M, N), dtype=torch.float32, device=DEV)
    A_ref = torch.empty((g.M, N), dtype=torch.int64, device=DEV) if is_max else None
    G.spmm_run(plan, Bd, C_ref, A_ref, N, red)
    torch.cuda.synchronize()
    C = torch.full((g.M, N), float("nan"), device=DEV)
    A = torch.full((g.M, N), -7, dtype=torch.int64, device=DEV) if is_max else None
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side, capture_error_mode="thread_local"):
        G.spmm_run(plan, Bd, C, A, N, red)
    log(f"{case}: captured, route {G.spmm_plan_info(plan)['route_lanes']} lanes")
    for rep in range(4):
        C.fill_(float("nan"))
        if A is not None:
            A.fill_(-7)
        x = torch.randn(1 << 20, device=DEV)
        _ = float(x.sum())                                  # eager work and a sync between replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(C.view(torch.int32), C_ref.view(torch.int32)), f"replay {rep} differs"
        if A is not None:
            assert torch.equal(A, A_ref), f"replay {rep}: argmax differs"
    check(orc, g, B, red, C.cpu().numpy(), None if A is None else A.cpu().numpy(), what=f"graph {case}")
    del graph
    G.spmm_plan_destroy(plan)

"""GPU parity of the V = 2 vectorized-blocking panels (option SPMM_OPT_VBLOCK)
through the C ABI.

Rows stored with ascending columns keep their stored order inside a panel,
so sum / mean are bit-exact against the oracle's fused mode and max / argmax
bit-exact; rows with unsorted columns are summed in ascending column order
(fp32 tolerance), and max then keeps the row kernels.  The panel count of
nonzero vectors is checked against a numpy count."""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gnn_sparse_dense_amd as G
    from tests.gpu_helpers import DEV, check, gpu_run, log, make_plan, to_dev


def expected_vectors(g):
    """Sum over (panel, column) of max(occurrences in row 2g, in row 2g+1)."""
    rows = np.repeat(np.arange(g.M), g.degrees())
    key = (rows // 2) * g.K + g.col
    k0, c0 = np.unique(key[rows % 2 == 0], return_counts=True)
    k1, c1 = np.unique(key[rows % 2 == 1], return_counts=True)
    allk = np.union1d(k0, k1)
    n0 = np.zeros(allk.size, np.int64)
    n1 = np.zeros(allk.size, np.int64)
    n0[np.searchsorted(allk, k0)] = c0
    n1[np.searchsorted(allk, k1)] = c1
    return int(np.maximum(n0, n1).sum())


def panel_plan(g, mode=2):
    plan = make_plan(g)
    G.spmm_plan_set_option(plan, G.SPMM_OPT_VBLOCK, mode)
    return plan


SORTED = [
    ("knn", lambda rng: W.knn_line(3001, 10)),
    ("sorted-dups", lambda rng: W.random_csr(rng, 2501, 1800, mean_deg=7.0, empty_frac=0.1, dup_frac=0.2)),
    ("sorted-unweighted", lambda rng: W.random_csr(rng, 1200, 900, mean_deg=5.0, weighted=False)),
    ("road", lambda rng: W.make_graph("road", M=20_000)),
]


@pytest.mark.parametrize("name,make", SORTED, ids=[c[0] for c in SORTED])
@pytest.mark.parametrize("N", [1, 13, 16, 64, 100, 256])
def test_panels_sorted_rows_bit_exact(orc, name, make, N):
    rng = np.random.default_rng(N)
    g = make(rng)
    B = rng.integers(-3, 4, size=(g.K, N)).astype(np.float32) if N == 13 else \
        rng.standard_normal((g.K, N)).astype(np.float32)
    log(f"panels {name} M={g.M} nnz={g.nnz} N={N}")
    plan = panel_plan(g)
    info = G.spmm_plan_info(plan)
    assert info["pairs_built"] == 1 and info["pair_vectors"] == expected_vectors(g)
    _, _, _, Bd = to_dev(g, B)
    for red in ("sum", "mean", "max"):
        C, arg = gpu_run(plan, g.M, Bd, red)
        assert G.spmm_plan_info(plan)["route_pairs"] == 1
        check(orc, g, B, red, C, arg, exact_rows=np.arange(g.M), what=f"{name} N={N} {red}")
    G.spmm_plan_destroy(plan)


def test_panels_unsorted_rows(orc):
    rng = np.random.default_rng(11)
    g = W.random_csr(rng, 3333, 2000, mean_deg=6.0, empty_frac=0.1, dup_frac=0.2, shuffle_rows=True)
    plan = panel_plan(g)
    info = G.spmm_plan_info(plan)
    assert info["pairs_built"] == 2 and info["pair_vectors"] == expected_vectors(g)
    B = rng.standard_normal((g.K, 48)).astype(np.float32)
    _, _, _, Bd = to_dev(g, B)
    for red in ("sum", "mean"):
        C, _ = gpu_run(plan, g.M, Bd, red)
        assert G.spmm_plan_info(plan)["route_pairs"] == 1
        check(orc, g, B, red, C, None, what=f"unsorted {red}")
    Bt = rng.integers(0, 3, size=(g.K, 48)).astype(np.float32)
    _, _, _, Btd = to_dev(g, Bt)
    C, arg = gpu_run(plan, g.M, Btd, "max")
    assert G.spmm_plan_info(plan)["route_pairs"] == 0          # tie order needs stored order
    check(orc, g, Bt, "max", C, arg, what="unsorted max (row kernels)")
    G.spmm_plan_destroy(plan)


def test_panels_auto_by_padding(orc):
    rng = np.random.default_rng(12)
    knn = W.knn_line(5000, 10)
    rnd = W.random_csr(rng, 5000, 5000, mean_deg=10.0, weighted=False)
    B = rng.standard_normal((5000, 32)).astype(np.float32)
    for g, want in ((knn, 1), (rnd, 0)):
        plan = panel_plan(g, mode=1)
        info = G.spmm_plan_info(plan)
        _, _, _, Bd = to_dev(g, B)
        C, _ = gpu_run(plan, g.M, Bd, "sum")
        info = G.spmm_plan_info(plan)
        log(f"auto: padding {info['pair_padding']:.3f} -> route_pairs {info['route_pairs']}")
        assert info["route_pairs"] == want
        check(orc, g, B, "sum", C, None, exact_rows=np.arange(g.M), what="auto")
        G.spmm_plan_set_option(plan, G.SPMM_OPT_VBLOCK, 0)
        assert G.spmm_plan_info(plan)["pairs_built"] == 0
        G.spmm_plan_destroy(plan)


def test_panels_degenerate(orc):
    rng = np.random.default_rng(13)
    cases = [
        W.Graph("one", 1, 5, np.array([0, 3]), np.array([0, 2, 4]), None),
        W.Graph("empty", 7, 4, np.zeros(8, np.int64), np.zeros(0, np.int64), None),
        W.Graph("k0", 3, 0, np.zeros(4, np.int64), np.zeros(0, np.int64), None),
        W.random_csr(rng, 9, 6, mean_deg=3.0, empty_frac=0.3),
    ]
    for g in cases:
        plan = panel_plan(g)
        B = rng.standard_normal((g.K, 8)).astype(np.float32)
        Bd = torch.from_numpy(B).to(DEV) if g.K else torch.zeros((0, 8), device=DEV)
        for red in ("sum", "mean", "max"):
            C, arg = gpu_run(plan, g.M, Bd, red)
            check(orc, g, B, red, C, arg, what=f"{g.name} {red}")
        G.spmm_plan_destroy(plan)


def test_panels_forced_lanes_and_determinism(orc):
    g = W.knn_line(4097, 16)
    rng = np.random.default_rng(14)
    B = rng.standard_normal((g.K, 64)).astype(np.float32)
    _, _, _, Bd = to_dev(g, B)
    plan = panel_plan(g)
    ref = None
    for lanes in (4, 8, 16, 32, 64):
        G.spmm_plan_set_option(plan, G.SPMM_OPT_LANES, lanes)
        C, _ = gpu_run(plan, g.M, Bd, "sum")
        assert G.spmm_plan_info(plan)["route_lanes"] == lanes
        if ref is None:
            ref = C
            check(orc, g, B, "sum", C, None, exact_rows=np.arange(g.M), what="forced lanes")
        assert np.array_equal(C.view(np.uint32), ref.view(np.uint32)), f"lanes={lanes} differs"
    G.spmm_plan_destroy(plan)


def test_panels_full_road_sampled(orc):
    w = W.make("road")
    g, B = w.graph, w.B
    plan = panel_plan(g)
    _, _, _, Bd = to_dev(g, B)
    C, _ = gpu_run(plan, g.M, Bd, "sum")
    info = G.spmm_plan_info(plan)
    log(f"road panels: vectors {info['pair_vectors']} padding {info['pair_padding']:.3f}")
    rows = np.unique(np.concatenate([np.linspace(0, g.M - 1, 500).astype(np.int64), np.arange(g.M - 30, g.M)]))
    check(orc, g, B, "sum", C[rows], None, rows=rows, exact_rows=np.arange(rows.size), what="road panels")
    G.spmm_plan_destroy(plan)


def test_panels_built_automatically(orc):
    """SPMM_OPT_VBLOCK = -1 (the default): plan creation builds the panels of a
    plan with sorted rows when their padding share is at most 0.3 (merge
    count and merge build, no sort); the vectors equal a numpy count and the
    products stay bit-exact.  Graphs with more padding, unsorted rows or a
    row split keep the row kernels."""
    rng = np.random.default_rng(15)
    cases = [
        ("knn", W.knn_line(6001, 10), 1),
        ("knn weighted dups", None, 1),
        ("random sorted", W.random_csr(rng, 5000, 5000, mean_deg=10.0, weighted=False), 0),
        ("random unsorted", W.random_csr(rng, 5000, 5000, mean_deg=10.0, shuffle_rows=True), 0),
    ]
    # a weighted kNN graph with every row's last column stored twice
    k = W.knn_line(4001, 8)
    deg = k.degrees()
    cols, vals, rp = [], [], [0]
    for i in range(k.M):
        c = list(k.col[k.rowptr[i]:k.rowptr[i + 1]])
        c = c + c[-1:]
        cols += c
        vals += list(rng.random(len(c)).astype(np.float32))
        rp.append(len(cols))
    cases[1] = ("knn weighted dups", W.Graph("kd", k.M, k.K, np.array(rp, np.int64), np.array(cols, np.int64),
                                             np.array(vals, np.float32)), 1)
    for name, g, want in cases:
        plan = make_plan(g)
        info = G.spmm_plan_info(plan)
        log(f"auto panels {name}: built {info['pairs_built']} padding {info['pair_padding']:.3f}")
        assert info["pairs_built"] == want, name
        if want:
            assert info["pair_vectors"] == expected_vectors(g) and info["pair_padding"] <= 0.3
        for N in (16, 64):
            B = rng.standard_normal((g.K, N)).astype(np.float32)
            _, _, _, Bd = to_dev(g, B)
            for red in ("sum", "mean", "max"):
                C, arg = gpu_run(plan, g.M, Bd, red)
                assert G.spmm_plan_info(plan)["route_pairs"] == want, (name, N, red)
                exact = np.arange(g.M) if name != "random unsorted" else None
                check(orc, g, B, red, C, arg, exact_rows=exact, what=f"auto {name} N={N} {red}")
        G.spmm_plan_destroy(plan)

"""GPU parity of merge-path balancing (option SPMM_OPT_BALANCE = 1) through
the C ABI.  Rows that lie inside one segment of 512 merge items (their first
entry and their end in the same segment) are summed in stored order with one
accumulator: bit-exact against the fused oracle; rows spread over segments
are folded piece by piece in order: fp32 tolerance.  Max and argmax are
bit-exact everywhere (ties forced across segment boundaries)."""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gnn_sparse_dense_amd as G
    from tests.gpu_helpers import DEV, check, gpu_run, log, make_plan, to_dev

D = 512


def whole_rows(g):
    r = np.arange(g.M)
    first = g.rowptr[:-1] + r            # merge position of the row's first entry
    end = g.rowptr[1:] + r               # merge position of the row's end item
    return np.nonzero(first // D == end // D)[0]


def merge_plan(g):
    plan = make_plan(g)
    G.spmm_plan_set_option(plan, G.SPMM_OPT_BALANCE, 1)
    info = G.spmm_plan_info(plan)
    assert info["merge_segments"] == (g.M + g.nnz + D - 1) // D
    return plan


GRAPHS = [
    ("skewed", lambda rng: W.random_csr(rng, 4000, 3000, mean_deg=6.0, empty_frac=0.2, dup_frac=0.1,
                                        shuffle_rows=True, heavy_rows=5, heavy_deg=3000)),
    ("powerlaw", lambda rng: W.make_graph("powerlaw", M=60_000)),
    ("road", lambda rng: W.make_graph("road", M=30_000)),
]


@pytest.mark.parametrize("name,make", GRAPHS, ids=[c[0] for c in GRAPHS])
@pytest.mark.parametrize("N", [1, 7, 64, 128, 300])
def test_merge_parity(orc, name, make, N):
    rng = np.random.default_rng(N + 3)
    g = make(rng)
    log(f"merge {name} M={g.M} nnz={g.nnz} N={N}")
    plan = merge_plan(g)
    exact = whole_rows(g)
    B = rng.standard_normal((g.K, N)).astype(np.float32)
    _, _, _, Bd = to_dev(g, B)
    for red in ("sum", "mean"):
        C, _ = gpu_run(plan, g.M, Bd, red)
        assert G.spmm_plan_info(plan)["route_merge"] == 1
        check(orc, g, B, red, C, None, exact_rows=exact, what=f"{name} N={N} {red}")
        C2, _ = gpu_run(plan, g.M, Bd, red)
        assert np.array_equal(C.view(np.uint32), C2.view(np.uint32)), "runs differ"
    Bt = rng.integers(0, 3, size=(g.K, N)).astype(np.float32)       # many ties
    _, _, _, Btd = to_dev(g, Bt)
    C, arg = gpu_run(plan, g.M, Btd, "max")
    check(orc, g, Bt, "max", C, arg, what=f"{name} N={N} max")
    G.spmm_plan_destroy(plan)


def test_merge_degenerate_and_option(orc):
    rng = np.random.default_rng(5)
    cases = [
        W.Graph("empty", 3000, 100, np.zeros(3001, np.int64), np.zeros(0, np.int64), None),
        W.Graph("one-long-row", 1, 5000, np.array([0, 20000]), rng.integers(0, 5000, 20000), None),
        W.Graph("long-row-then-empty", 700, 900,
                np.concatenate([[0], np.full(700, 5000)]).astype(np.int64), rng.integers(0, 900, 5000),
                rng.random(5000, dtype=np.float32)),
        W.random_csr(rng, 3, 4, mean_deg=2.0),
    ]
    for g in cases:
        plan = merge_plan(g)
        B = rng.standard_normal((g.K, 20)).astype(np.float32)
        _, _, _, Bd = to_dev(g, B)
        for red in ("sum", "mean", "max"):
            C, arg = gpu_run(plan, g.M, Bd, red)
            check(orc, g, B, red, C, arg, exact_rows=(whole_rows(g) if red != "max" else None),
                  what=f"{g.name} {red}")
        G.spmm_plan_set_option(plan, G.SPMM_OPT_BALANCE, 0)
        info = G.spmm_plan_info(plan)
        assert info["merge_segments"] == 0
        C, _ = gpu_run(plan, g.M, Bd, "sum")
        assert G.spmm_plan_info(plan)["route_merge"] == 0
        G.spmm_plan_destroy(plan)


def test_merge_full_powerlaw_sampled(orc):
    w = W.make("powerlaw")
    g, B = w.graph, w.B
    plan = merge_plan(g)
    _, _, _, Bd = to_dev(g, B)
    C, _ = gpu_run(plan, g.M, Bd, "sum")
    deg = g.degrees()
    rows = np.unique(np.concatenate([np.linspace(0, g.M - 1, 400).astype(np.int64),
                                     np.argsort(deg)[-40:], np.arange(g.M - 20, g.M)]))
    check(orc, g, B, "sum", C[rows], None, rows=rows, what="full power-law (sampled rows)")
    G.spmm_plan_destroy(plan)


@pytest.mark.parametrize("N", [257, 259, 302, 513, 602])
def test_merge_float4_at_any_width(orc, N):
    """Merge path on float4 lanes at widths that are not a multiple of 4 (a
    row's last vector moved back to end at column N; a last 256-column pass of
    fewer than 4 columns starts earlier), and with B and C one element past an
    allocation's start: sum and mean in tolerance (whole rows bit-exact), max
    and argmax bit-exact."""
    rng = np.random.default_rng(N + 11)
    g = W.make_graph("road", M=30_000)
    plan = merge_plan(g)
    exact = whole_rows(g)
    B = rng.standard_normal((g.K, N)).astype(np.float32)
    _, _, _, Bd = to_dev(g, B)
    for red in ("sum", "mean", "max"):
        log(f"merge float4 N={N} {red}")
        C, arg = gpu_run(plan, g.M, Bd, red)
        info = G.spmm_plan_info(plan)
        assert info["route_merge"] == 1 and info["route_vec"] == 4, info
        check(orc, g, B, red, C, arg, exact_rows=exact, what=f"merge N={N} {red}")
    Bbig = torch.empty(g.K * N + 1, dtype=torch.float32, device=DEV)
    Bv = Bbig[1:].view(g.K, N)
    Bv.copy_(Bd)
    Cbig = torch.full((g.M * N + 2,), float("nan"), dtype=torch.float32, device=DEV)
    Cv = Cbig[1:-1].view(g.M, N)
    G.spmm_run(plan, Bv, Cv, None, N, "sum", None)
    torch.cuda.synchronize()
    assert G.spmm_plan_info(plan)["route_vec"] == 4
    assert np.isnan(Cbig[0].item()) and np.isnan(Cbig[-1].item())
    check(orc, g, B, "sum", Cv.cpu().numpy(), None, exact_rows=exact, what=f"merge offset N={N}")
    G.spmm_plan_destroy(plan)

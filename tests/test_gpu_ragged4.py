"""GPU parity of float4 lanes on rows that are only 4-byte aligned.

When N is not a multiple of 4, or B, C or argmax start at an offset, every
B and C row still takes 16-byte accesses per lane: the one vector that would
run past column N is moved back to end at N, and the columns it shares with
its neighbour lane are computed by both with the same bits.  These tests run
that path on every kernel that takes it (row kernel, row tiles, split pieces
with one or two dispatches, V = 2 panels) against the oracle, and check it
bit for bit against forced float1 lanes.
"""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gnn_sparse_dense_amd as G
    from tests.gpu_helpers import DEV, check, gpu_run, log, make_plan, to_dev

WIDTHS = (4, 5, 6, 7, 9, 13, 33, 66, 130, 257, 258, 259, 602)


def _graph(kind, rng):
    if kind == "rows":
        return W.random_csr(rng, 1800, 1500, mean_deg=9.0, empty_frac=0.05, dup_frac=0.05, shuffle_rows=True)
    if kind == "tiles":
        return W.make_graph("road", M=6000)
    if kind == "split":
        return W.random_csr(rng, 2000, 1700, mean_deg=6.0, empty_frac=0.05, heavy_rows=5, heavy_deg=1500)
    if kind == "window_sorted":     # sorted rows: the three-run window kernel
        return W.make_graph("community", M=3072)
    if kind == "window":            # unsorted rows: the per-entry window kernel
        return W.block_csr(rng, 2500, 2500, in_deg=12.0, off_deg=2.0)
    return W.knn_line(3000, 10)


@pytest.mark.parametrize("kind", ["rows", "tiles", "split", "panels", "window_sorted", "window"])
def test_ragged_float4_widths(orc, kind):
    rng = np.random.default_rng(404)
    g = _graph(kind, rng)
    # float4 lanes forced: the router takes float1 lanes for some of these
    # widths on graphs this small
    plan = make_plan(g, [(G.SPMM_OPT_VEC, 4)])
    if kind == "split":
        assert G.spmm_plan_info(plan)["n_heavy"] > 0
    exact = G.spmm_plan_partition(plan)["light"] if kind == "split" else np.arange(g.M)
    for N in WIDTHS:
        B = rng.standard_normal((g.K, N)).astype(np.float32)
        _, _, _, Bd = to_dev(g, B)
        for red in ("sum", "mean", "max"):
            what = f"{kind} N={N} {red}"
            log(what)
            C, arg = gpu_run(plan, g.M, Bd, red)
            info = G.spmm_plan_info(plan)
            assert info["route_vec"] == 4, (what, info)
            if kind == "tiles" and N <= 32:
                assert info["route_tiled"] == 1, (what, info)
            if kind == "panels" and red != "max":
                assert info["route_pairs"] == 1 or N >= 128, (what, info)
            if kind.startswith("window") and N > 32:
                assert info["route_window"] == (2 if kind == "window_sorted" else 1), (what, info)
            check(orc, g, B, red, C, arg, exact_rows=exact, what=what)
    G.spmm_plan_destroy(plan)


@pytest.mark.parametrize("N", [5, 33, 130, 259])
def test_ragged_float4_matches_float1_bitwise(orc, N):
    """Forced float1 lanes and the float4 route give the same bits."""
    rng = np.random.default_rng(500 + N)
    g = W.random_csr(rng, 2500, 2000, mean_deg=8.0, empty_frac=0.05, dup_frac=0.1, shuffle_rows=True,
                     heavy_rows=4, heavy_deg=900)
    B = rng.standard_normal((g.K, N)).astype(np.float32)
    _, _, _, Bd = to_dev(g, B)
    for red in ("sum", "mean", "max"):
        outs = []
        for vec in (1, 4):
            for fused in (0, 1):
                plan = make_plan(g, [(G.SPMM_OPT_VEC, vec), (G.SPMM_OPT_SPLIT_FUSED, fused)])
                log(f"N={N} {red} vec={vec} fused={fused}")
                C, arg = gpu_run(plan, g.M, Bd, red)
                assert G.spmm_plan_info(plan)["route_vec"] == vec
                outs.append((C, arg))
                G.spmm_plan_destroy(plan)
        for C, arg in outs[1:]:
            assert np.array_equal(C.view(np.uint32), outs[0][0].view(np.uint32)), (N, red)
            if arg is not None:
                assert np.array_equal(arg, outs[0][1]), (N, red)
        check(orc, g, B, red, outs[0][0], outs[0][1], what=f"N={N} {red}")


@pytest.mark.parametrize("N", [33, 64])
def test_offset_pointers(orc, N):
    """B and C one float past a 16-byte boundary and argmax one int64 past it:
    the float4 route with 4-byte aligned rows, bit-exact with the aligned run."""
    rng = np.random.default_rng(600 + N)
    g = W.random_csr(rng, 9000, 8000, mean_deg=7.0, empty_frac=0.05)
    B = rng.standard_normal((g.K, N)).astype(np.float32)
    plan = make_plan(g)
    _, _, _, Bd = to_dev(g, B)
    Bbig = torch.empty(g.K * N + 1, dtype=torch.float32, device=DEV)
    Bv = Bbig[1:].view(g.K, N)
    Bv.copy_(Bd)
    for red in ("sum", "mean", "max"):
        log(f"offset pointers N={N} {red}")
        Cbig = torch.full((g.M * N + 2,), float("nan"), dtype=torch.float32, device=DEV)
        Cv = Cbig[1:-1].view(g.M, N)
        Abig = None
        Av = None
        if red == "max":
            Abig = torch.full((g.M * N + 2,), 0x7F7F7F7F7F7F7F7F, dtype=torch.int64, device=DEV)
            Av = Abig[1:-1].view(g.M, N)
        G.spmm_run(plan, Bv, Cv, Av, N, red, None)
        torch.cuda.synchronize()
        assert G.spmm_plan_info(plan)["route_vec"] == 4
        C = Cv.cpu().numpy()
        arg = None if Av is None else Av.cpu().numpy()
        assert np.isnan(Cbig[0].item()) and np.isnan(Cbig[-1].item()), "a float next to C was written"
        if Abig is not None:
            assert Abig[0].item() == 0x7F7F7F7F7F7F7F7F and Abig[-1].item() == 0x7F7F7F7F7F7F7F7F, \
                "an int64 next to argmax was written"
        check(orc, g, B, red, C, arg, exact_rows=np.arange(g.M), what=f"offset N={N} {red}")
        Ca, arga = gpu_run(plan, g.M, Bd, red)
        assert np.array_equal(C.view(np.uint32), Ca.view(np.uint32))
        if arg is not None:
            assert np.array_equal(arg, arga)
    G.spmm_plan_destroy(plan)


@pytest.mark.parametrize("N", [257, 258, 259, 513])
def test_split_last_pass_narrower_than_a_vector(orc, N):
    """Split rows at widths whose last 256-column pass holds 1 to 3 columns:
    that pass starts earlier so that its vectors stay inside it."""
    rng = np.random.default_rng(700 + N)
    g = W.random_csr(rng, 1500, 1400, mean_deg=5.0, empty_frac=0.05, heavy_rows=6, heavy_deg=1200)
    B = rng.standard_normal((g.K, N)).astype(np.float32)
    plan = make_plan(g)
    assert G.spmm_plan_info(plan)["n_heavy"] > 0
    light = G.spmm_plan_partition(plan)["light"]
    _, _, _, Bd = to_dev(g, B)
    for red in ("sum", "mean", "max"):
        log(f"split last pass N={N} {red}")
        C, arg = gpu_run(plan, g.M, Bd, red)
        assert G.spmm_plan_info(plan)["route_vec"] == 4
        check(orc, g, B, red, C, arg, exact_rows=light, what=f"split N={N} {red}")
    G.spmm_plan_destroy(plan)


def test_router_ragged_rules():
    """Routing at widths that are not a multiple of 4 (measured with the
    router sweep): float4 lanes by default; float1 lanes for rows of at most
    8 floats at mean degree 16 and above, of at most 16 floats on split
    skewed graphs and below 128 floats on small graphs; half the lane group, coarsened, for 17 to 63 vectors that leave a quarter of it
    idle at mean degree below 16; skewed graphs without column slices at such
    widths; V = 2 panels with 64 lanes past 32 vectors; the window kernel for
    community structure from 33 floats."""
    diffusion = make_plan(W.make_graph("diffusion", M=100_000))
    for N, want in ((33, (4, 16, 1)), (66, (4, 16, 2)), (130, (4, 32, 2)), (602, (4, 64, 2)), (7, (4, 4, 1))):
        info = G.spmm_plan_route(diffusion, N, "sum")
        assert (info["route_vec"], info["route_lanes"], info["route_coarsen"]) == want, (N, info)
    G.spmm_plan_destroy(diffusion)
    community = make_plan(W.make_graph("community", M=20_000))
    info = G.spmm_plan_route(community, 7, "sum")
    assert (info["route_vec"], info["route_lanes"]) == (1, 8), info
    for N in (33, 66, 130, 602):
        assert G.spmm_plan_route(community, N, "sum")["route_window"] > 0, N
    assert G.spmm_plan_route(community, 17, "sum")["route_window"] == 0
    G.spmm_plan_destroy(community)
    tiny = make_plan(W.make_graph("tiny"))
    assert G.spmm_plan_route(tiny, 33, "sum")["route_vec"] == 1
    assert G.spmm_plan_route(tiny, 130, "sum")["route_vec"] == 4
    G.spmm_plan_destroy(tiny)
    rng = np.random.default_rng(5)
    skew = make_plan(W.random_csr(rng, 20_000, 20_000, mean_deg=6.0, heavy_rows=20, heavy_deg=5000))
    assert G.spmm_plan_info(skew)["n_heavy"] > 0
    for N, want in ((130, (4, 64, 1, 1)), (258, (4, 64, 2, 1)), (128, (4, 16, 1, 2)), (16, (1, 16, 1, 1)),
                    (7, (1, 8, 1, 1)), (17, (4, 8, 1, 1))):
        info = G.spmm_plan_route(skew, N, "sum")
        got = (info["route_vec"], info["route_lanes"], info["route_coarsen"], info["route_slices"])
        assert got == want, (N, info)
    G.spmm_plan_destroy(skew)
    knn = make_plan(W.knn_line(50_000, 10))
    info = G.spmm_plan_route(knn, 130, "sum")
    assert (info["route_pairs"], info["route_lanes"]) == (1, 64), info
    assert G.spmm_plan_route(knn, 602, "sum")["route_window"] > 0
    G.spmm_plan_destroy(knn)


@pytest.mark.parametrize("N", [33, 64])
def test_forced_window_keeps_float4_on_small_graphs(orc, N):
    """The window kernels need float4 lanes: forcing them on a graph small
    enough for the router's float1 rule still routes them, with the oracle's
    results."""
    g = W.make_graph("community", M=3072)
    rng = np.random.default_rng(900 + N)
    B = rng.standard_normal((g.K, N)).astype(np.float32)
    plan = make_plan(g, [(G.SPMM_OPT_WINDOW, 1)])
    _, _, _, Bd = to_dev(g, B)
    for red in ("sum", "max"):
        log(f"forced window, small graph, N={N} {red}")
        C, arg = gpu_run(plan, g.M, Bd, red)
        info = G.spmm_plan_info(plan)
        assert info["route_window"] == 2 and info["route_vec"] == 4, info
        check(orc, g, B, red, C, arg, exact_rows=np.arange(g.M), what=f"forced window N={N} {red}")
    auto = make_plan(g)
    assert G.spmm_plan_route(auto, N, "sum")["route_vec"] == 1   # the small-graph rule
    G.spmm_plan_destroy(auto)
    G.spmm_plan_destroy(plan)


FULL_RAGGED = [("road", 33, "sum"), ("diffusion", 17, "max"), ("community", 130, "sum"), ("powerlaw", 130, "sum")]


@pytest.mark.parametrize("name,N,red", FULL_RAGGED, ids=[f[0] for f in FULL_RAGGED])
def test_full_size_ragged_widths_sampled(orc, name, N, red):
    """The full-size graphs at widths that are not a multiple of 4, in the
    router's own launch configuration: every output written, sampled rows
    against the oracle (evenly spaced, first and last, the longest rows and
    split rows; whole rows bit-exact)."""
    g = W.make_graph(name)
    rng = np.random.default_rng(1000 + N)
    B = rng.standard_normal((g.K, N)).astype(np.float32)
    log(f"full {name}: M={g.M} nnz={g.nnz} N={N} {red}")
    plan = make_plan(g)
    part = G.spmm_plan_partition(plan)
    _, _, _, Bd = to_dev(g, B)
    C, arg = gpu_run(plan, g.M, Bd, red, poison=True)
    info = G.spmm_plan_info(plan)
    assert info["route_vec"] == 4, info
    assert not np.isnan(C).any(), "unwritten output"
    deg = g.degrees()
    sample = np.unique(np.concatenate([
        np.arange(0, 64), np.arange(g.M - 64, g.M), rng.choice(g.M, size=2000, replace=False),
        np.argsort(deg)[-200:], np.unique(part["seg_row"])[:1000],
    ])).astype(np.int64)
    light_set = np.setdiff1d(sample, np.unique(part["seg_row"]))
    exact_idx = np.searchsorted(sample, light_set)
    check(orc, g, B, red, C[sample], None if arg is None else arg[sample], rows=sample, exact_rows=exact_idx,
          what=f"full {name} N={N} {red}")
    G.spmm_plan_destroy(plan)

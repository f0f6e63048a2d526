"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Sum and mean: |GPU - oracle| <= 1e-5 * sum|a*b| + 1e-6 per element; rows walked
whole are also bit-exact against the oracle's fused mode.  Max and argmax:
bit-exact.  Row split pieces: bit-exact against the oracle's partition.
"""
import functools

import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gnn_sparse_dense_amd as G
    from tests.gpu_helpers import DEV, check, gpu_run, log, make_plan, to_dev


@functools.lru_cache(maxsize=2)
def _workload(name, M=None):
    return W.make(name, M=M)


def _light_rows(plan, M):
    return G.spmm_plan_partition(plan)["light"]


def test_tiny_config_all_reductions(orc):
    w = _workload("tiny")
    g = w.graph
    log(f"tiny: M={g.M} nnz={g.nnz} N={w.N}")
    plan = make_plan(g)
    _, _, _, Bd = to_dev(g, w.B)
    for red in ("sum", "mean", "max"):
        C, arg = gpu_run(plan, g.M, Bd, red)
        check(orc, g, w.B, red, C, arg, exact_rows=np.arange(g.M), what=f"tiny {red}")
    G.spmm_plan_destroy(plan)


VARIANTS = [(lanes, coarsen, vec) for lanes in (4, 8, 16, 32, 64) for coarsen in (1, 2) for vec in (1, 2, 4)]


@pytest.mark.parametrize("weighted", [True, False])
def test_forced_variants_agree_bitwise(orc, weighted):
    rng = np.random.default_rng(101)
    g = W.random_csr(rng, 3001, 2500, mean_deg=9.0, empty_frac=0.05, dup_frac=0.1,
                     shuffle_rows=True, weighted=weighted, zero_frac=0.05)
    for N in (16, 64, 100, 37):
        B = rng.standard_normal((g.K, N)).astype(np.float32)
        _, _, _, Bd = to_dev(g, B)
        for red in ("sum", "mean", "max"):
            ref_out = None
            for lanes, coarsen, vec in VARIANTS:
                if vec == 2 and N % 2:   # float4 lanes also serve widths that are not a multiple of 4
                    continue
                what = f"N={N} {red} lanes={lanes} F={coarsen} vec={vec} w={weighted}"
                log(what)
                plan = make_plan(g, [(G.SPMM_OPT_LANES, lanes), (G.SPMM_OPT_COARSEN, coarsen),
                                     (G.SPMM_OPT_VEC, vec)])
                C, arg = gpu_run(plan, g.M, Bd, red)
                info = G.spmm_plan_info(plan)
                assert (info["route_lanes"], info["route_coarsen"], info["route_vec"]) == (lanes, coarsen, vec)
                if ref_out is None:
                    check(orc, g, B, red, C, arg, exact_rows=np.arange(g.M), what=what)
                    ref_out = (C, arg)
                else:
                    assert np.array_equal(C.view(np.uint32), ref_out[0].view(np.uint32)), what
                    if arg is not None:
                        assert np.array_equal(arg, ref_out[1]), what
                G.spmm_plan_destroy(plan)


@pytest.mark.parametrize("N", [1, 3, 17, 63, 65, 100, 130, 257, 300, 1030])
def test_ragged_widths(orc, N):
    rng = np.random.default_rng(200 + N)
    g = W.random_csr(rng, 1500, 1200, mean_deg=7.0, empty_frac=0.1, dup_frac=0.05)
    B = rng.standard_normal((g.K, N)).astype(np.float32)
    plan = make_plan(g)
    _, _, _, Bd = to_dev(g, B)
    for red in ("sum", "mean", "max"):
        log(f"ragged N={N} {red}")
        C, arg = gpu_run(plan, g.M, Bd, red)
        check(orc, g, B, red, C, arg, exact_rows=np.arange(g.M), what=f"N={N} {red}")
    # an offset (8-byte but not 16-byte aligned) view of B: float4 lanes on
    # 4-byte aligned rows (float1 below 128 floats on this small graph)
    if N % 4 == 0:
        Bbig = torch.empty(g.K * N + 2, dtype=torch.float32, device=DEV)
        Bv = Bbig[2:].view(g.K, N)
        Bv.copy_(Bd)
        C, _ = gpu_run(plan, g.M, Bv, "sum")
        assert G.spmm_plan_info(plan)["route_vec"] == (1 if N < 128 else 4)
        check(orc, g, B, "sum", C, None, exact_rows=np.arange(g.M), what=f"N={N} misaligned B")
    G.spmm_plan_destroy(plan)


@pytest.mark.parametrize("route", ["rows", "tiles", "split", "split_fused", "window"])
def test_max_with_infinite_products(orc, route):
    """Finite inputs whose products overflow to -inf: weights 1e30 times B
    entries of -1e30 in half of B's columns.  Some rows hold only such
    entries (their max is -inf and their argmax the first entry), some start
    with them and continue with finite products, the rest are ordinary.  The
    max kernels start from -inf and take strictly larger values, then give
    an all -inf output its first entry: the oracle's stored-order rule."""
    rng = np.random.default_rng(71)
    g = W.random_csr(rng, 3000, 2048, mean_deg=9.0, empty_frac=0.05, dup_frac=0.1,
                     shuffle_rows=route != "window", weighted=True,
                     heavy_rows=6 if route.startswith("split") else 0,
                     heavy_deg=700)
    deg = g.degrees()
    all_inf = rng.choice(np.flatnonzero(deg > 0), size=300, replace=False)
    all_inf = np.union1d(all_inf, np.flatnonzero(deg == 700)[:3])   # split rows: every piece all -inf
    lead_inf = rng.choice(np.setdiff1d(np.flatnonzero(deg > 2), all_inf), size=300, replace=False)
    for i in all_inf:
        g.val[g.rowptr[i]:g.rowptr[i + 1]] = 1e30
    for i in lead_inf:
        g.val[g.rowptr[i]:g.rowptr[i] + 2] = 1e30
    N = {"window": 128, "split_fused": 64}.get(route, 24)
    B = rng.standard_normal((g.K, N)).astype(np.float32)
    B[:, ::2] = -1e30
    opts = {"rows": [(G.SPMM_OPT_TILES, 0)], "tiles": [(G.SPMM_OPT_TILES, 1)],
            "split": [(G.SPMM_OPT_SPLIT_T, 64), (G.SPMM_OPT_SPLIT_L, 50), (G.SPMM_OPT_SPLIT_MODE, 1)],
            "split_fused": [(G.SPMM_OPT_SPLIT_T, 64), (G.SPMM_OPT_SPLIT_L, 50), (G.SPMM_OPT_SPLIT_MODE, 1),
                            (G.SPMM_OPT_TILES, 0), (G.SPMM_OPT_LANES, 16), (G.SPMM_OPT_VEC, 4),
                            (G.SPMM_OPT_COARSEN, 1)],
            "window": [(G.SPMM_OPT_WINDOW, 1)]}[route]
    plan = make_plan(g, opts)
    _, _, _, Bd = to_dev(g, B)
    C, arg = gpu_run(plan, g.M, Bd, "max")
    info = G.spmm_plan_info(plan)
    routed = {"rows": info["route_tiled"] == 0 and info["route_window"] == 0,
              "tiles": info["route_tiled"] == 1, "split": info["n_heavy"] > 0,
              "split_fused": info["n_heavy"] > 0 and info["route_fused_split"] == 1,
              "window": info["route_window"] > 0}[route]
    assert routed, f"{route} not taken: {info}"
    assert np.isneginf(C[all_inf][:, ::2]).all()
    check(orc, g, B, "max", C, arg, what=f"-inf products, {route}")
    G.spmm_plan_destroy(plan)


def test_ties_and_signed_zeros(orc):
    rng = np.random.default_rng(7)
    for weighted in (False, True):
        g = W.random_csr(rng, 2000, 300, mean_deg=12.0, empty_frac=0.1, dup_frac=0.3,
                         shuffle_rows=True, weighted=weighted)
        if weighted:
            g.val = rng.choice(np.float32([0.0, -0.0, 0.5, 1.0, -1.0]), size=g.nnz).astype(np.float32)
        B = rng.integers(-1, 2, size=(g.K, 24)).astype(np.float32)
        B[rng.random(B.shape) < 0.2] = -0.0
        plan = make_plan(g)
        _, _, _, Bd = to_dev(g, B)
        for red in ("max", "sum", "mean"):
            C, arg = gpu_run(plan, g.M, Bd, red)
            check(orc, g, B, red, C, arg, exact_rows=np.arange(g.M), what=f"ties {red} w={weighted}")
        G.spmm_plan_destroy(plan)


def test_degenerate_shapes(orc):
    rng = np.random.default_rng(9)
    cases = [
        ("all empty", W.Graph("e", 50, 40, np.zeros(51, np.int64), np.zeros(0, np.int64), None)),
        ("K=0", W.Graph("k0", 7, 0, np.zeros(8, np.int64), np.zeros(0, np.int64), None)),
        ("one row", W.random_csr(rng, 1, 500, mean_deg=300.0, empty_frac=0.0)),
        ("one long row", W.random_csr(rng, 3, 100, mean_deg=2.0, empty_frac=0.0, heavy_rows=1,
                                      heavy_deg=5000)),
        ("identity", W.Graph("i", 333, 333, np.arange(334, dtype=np.int64), np.arange(333, dtype=np.int64),
                             None)),
    ]
    for what, g in cases:
        N = 20
        B = rng.standard_normal((g.K, N)).astype(np.float32)
        log(f"degenerate: {what}")
        plan = make_plan(g)
        if g.K == 0:
            Bd = torch.empty((0, N), dtype=torch.float32, device=DEV)
        else:
            _, _, _, Bd = to_dev(g, B)
        for red in ("sum", "mean", "max"):
            C, arg = gpu_run(plan, g.M, Bd, red)
            if g.K == 0:
                assert np.all(C.view(np.uint32) == 0) and (arg is None or np.all(arg == -1))
                continue
            check(orc, g, B, red, C, arg, exact_rows=None, what=f"{what} {red}")
        G.spmm_plan_destroy(plan)
    # M = 0: a no-op
    g0 = W.Graph("m0", 0, 5, np.zeros(1, np.int64), np.zeros(0, np.int64), None)
    plan = make_plan(g0)
    Bd = torch.zeros((5, 4), dtype=torch.float32, device=DEV)
    C = torch.empty((0, 4), dtype=torch.float32, device=DEV)
    G.spmm_run(plan, Bd, C, None, 4, "sum")
    torch.cuda.synchronize()
    G.spmm_plan_destroy(plan)


def test_size_limits(orc):
    # rowptr[M] at the int32 limit is refused from rowptr alone: col is never read
    rp = torch.tensor([0, 2**31 - 1], dtype=torch.int64, device=DEV)
    cl = torch.zeros(1, dtype=torch.int64, device=DEV)
    assert G.lib().spmm_plan_create(rp.data_ptr(), cl.data_ptr(), None, 1, 4) is None
    st, msg = G.spmm_last_error()
    assert st == G.SPMM_E_UNSUPPORTED and "nnz" in msg
    # the binding refuses the same arrays earlier: col is shorter than rowptr[M]
    with pytest.raises(ValueError, match="col has 1 elements"):
        G.spmm_plan_create(rp, cl, None, 1, 4)
    # very wide feature rows: hundreds of column slices with a ragged last one
    rng = np.random.default_rng(12)
    g = W.random_csr(rng, 40, 30, mean_deg=6.0, empty_frac=0.1, heavy_rows=1, heavy_deg=25,
                     dup_frac=0.1)
    plan = make_plan(g)
    for N in (20_001, 65_540):
        log(f"wide N={N}")
        B = rng.standard_normal((g.K, N)).astype(np.float32)
        _, _, _, Bd = to_dev(g, B)
        for red in ("sum", "mean", "max"):
            C, arg = gpu_run(plan, g.M, Bd, red)
            check(orc, g, B, red, C, arg, exact_rows=None, what=f"wide N={N} {red}")
    G.spmm_plan_destroy(plan)


@pytest.mark.parametrize("T,L", [(64, 64), (100, 37), (0, 1000), (513, 512)])
def test_row_split(orc, T, L):
    rng = np.random.default_rng(T * 7 + L)
    g = W.random_csr(rng, 4000, 3000, mean_deg=6.0, empty_frac=0.05, heavy_rows=25, heavy_deg=2100,
                     dup_frac=0.05, shuffle_rows=True)
    plan = make_plan(g, [(G.SPMM_OPT_SPLIT_T, T), (G.SPMM_OPT_SPLIT_L, L), (G.SPMM_OPT_SPLIT_MODE, 1)])
    part = G.spmm_plan_partition(plan)
    ref = orc.partition(g.rowptr, g.M, T, L)
    log(f"split T={T} L={L}: heavy={part['n_heavy']} pieces={len(part['seg_row'])}")
    assert part["n_heavy"] == ref["n_heavy"] > 0
    for k in ("seg_row", "seg_begin", "seg_end", "light"):
        assert np.array_equal(part[k], ref[k]), k
    info = G.spmm_plan_info(plan)
    assert info["split_T"] == T and info["split_L"] == L and info["n_seg"] == len(ref["seg_row"])
    for N in (48, 130, 300):
        B = rng.standard_normal((g.K, N)).astype(np.float32)
        _, _, _, Bd = to_dev(g, B)
        for red in ("sum", "mean", "max"):
            C, arg = gpu_run(plan, g.M, Bd, red)
            check(orc, g, B, red, C, arg, exact_rows=ref["light"], what=f"split T={T} L={L} N={N} {red}")
    G.spmm_plan_destroy(plan)


@pytest.mark.parametrize("shuffled", [False, True], ids=["sorted-rows", "shuffled-rows"])
def test_piece_order_same_bits(orc, shuffled):
    """The split's pieces run in the order of their first entry's column by
    default: the partition it reports is unchanged, and every output bit
    equals that of the pieces run in partition order (sum, mean, max and
    argmax, column passes of 256 and a ragged tail)."""
    rng = np.random.default_rng(9090 + shuffled)
    g = W.random_csr(rng, 6000, 50_000, mean_deg=5.0, empty_frac=0.05, heavy_rows=60, heavy_deg=4000,
                     dup_frac=0.02, shuffle_rows=shuffled)
    opts = [(G.SPMM_OPT_SPLIT_T, 256), (G.SPMM_OPT_SPLIT_L, 200), (G.SPMM_OPT_SPLIT_MODE, 1)]
    on = make_plan(g, opts)
    off = make_plan(g, opts + [(G.SPMM_OPT_PIECE_ORDER, 0)])
    assert G.spmm_plan_info(on)["piece_order"] == 1
    assert G.spmm_plan_info(off)["piece_order"] == 0
    p_on, p_off = G.spmm_plan_partition(on), G.spmm_plan_partition(off)
    ref = orc.partition(g.rowptr, g.M, 256, 200)
    for k in ("seg_row", "seg_begin", "seg_end", "light"):
        assert np.array_equal(p_on[k], ref[k]) and np.array_equal(p_off[k], ref[k]), k
    for N in (64, 300):
        B = rng.standard_normal((g.K, N)).astype(np.float32)
        _, _, _, Bd = to_dev(g, B)
        for red in ("sum", "mean", "max"):
            C1, a1 = gpu_run(on, g.M, Bd, red)
            C0, a0 = gpu_run(off, g.M, Bd, red)
            log(f"piece order shuffled={shuffled} N={N} {red}")
            assert np.array_equal(C1.view(np.uint32), C0.view(np.uint32)), f"N={N} {red}"
            if red == "max":
                assert np.array_equal(a1, a0)
            check(orc, g, B, red, C1, a1, exact_rows=ref["light"], what=f"piece order N={N} {red}")
    # switching the option rebuilds the split in place
    G.spmm_plan_set_option(off, G.SPMM_OPT_PIECE_ORDER, 1)
    assert G.spmm_plan_info(off)["piece_order"] == 1
    G.spmm_plan_destroy(on)
    G.spmm_plan_destroy(off)


@pytest.mark.parametrize("weighted", [True, False])
def test_split_fused_same_bits(orc, weighted):
    """A split product of at most 256 columns on the row kernel runs its light
    rows and its pieces in one dispatch by default: every output bit equals
    that of the two dispatches (sum, mean, max and argmax), with the router's
    launch shape and with forced 16- and 32-lane shapes, XCD remap on and
    off; wider products keep two dispatches."""
    rng = np.random.default_rng(4242 + weighted)
    g = W.random_csr(rng, 20_000, 20_000, mean_deg=6.0, empty_frac=0.05, heavy_rows=40, heavy_deg=5000,
                     dup_frac=0.01, shuffle_rows=True, weighted=weighted)
    shapes = [[], [(G.SPMM_OPT_LANES, 16), (G.SPMM_OPT_VEC, 4), (G.SPMM_OPT_COARSEN, 1), (G.SPMM_OPT_XCD_REMAP, 1)],
              [(G.SPMM_OPT_LANES, 32), (G.SPMM_OPT_VEC, 4), (G.SPMM_OPT_COARSEN, 1), (G.SPMM_OPT_XCD_REMAP, 0)]]
    light = None
    for si, shape in enumerate(shapes):
        on = make_plan(g, shape)
        off = make_plan(g, shape + [(G.SPMM_OPT_SPLIT_FUSED, 0)])
        assert G.spmm_plan_info(on)["n_seg"] > 0
        if light is None:
            light = _light_rows(on, g.M)
        for N in (32, 128, 256, 300):
            B = rng.standard_normal((g.K, N)).astype(np.float32)
            _, _, _, Bd = to_dev(g, B)
            for red in ("sum", "mean", "max"):
                what = f"split fused shape={si} N={N} {red} w={weighted}"
                log(what)
                C1, a1 = gpu_run(on, g.M, Bd, red)
                i1 = G.spmm_plan_info(on)
                C0, a0 = gpu_run(off, g.M, Bd, red)
                assert G.spmm_plan_info(off)["route_fused_split"] == 0
                can = (i1["route_lanes"] in (16, 32) and i1["route_vec"] == 4 and i1["route_coarsen"] == 1
                       and not i1["route_window"] and not i1["route_tiled"] and N <= 256)
                assert i1["route_fused_split"] == int(can), (what, i1)
                if si > 0 and N <= 256:
                    assert can, (what, i1)
                assert np.array_equal(C1.view(np.uint32), C0.view(np.uint32)), what
                if red == "max":
                    assert np.array_equal(a1, a0), what
                if si == 0:
                    check(orc, g, B, red, C1, a1, exact_rows=light, what=what)
        G.spmm_plan_destroy(on)
        G.spmm_plan_destroy(off)


def test_split_fused_powerlaw_same_bits(orc):
    w = _workload("powerlaw", M=200_000)
    g = w.graph
    on, off = make_plan(g), make_plan(g, [(G.SPMM_OPT_SPLIT_FUSED, 0)])
    _, _, _, Bd = to_dev(g, w.B)
    for red in ("sum", "max"):
        log(f"split fused powerlaw M={g.M} N={w.N} {red}")
        C1, a1 = gpu_run(on, g.M, Bd, red)
        assert G.spmm_plan_info(on)["route_fused_split"] == 1
        C0, a0 = gpu_run(off, g.M, Bd, red)
        assert np.array_equal(C1.view(np.uint32), C0.view(np.uint32)), red
        if red == "max":
            assert np.array_equal(a1, a0)
    G.spmm_plan_destroy(on)
    G.spmm_plan_destroy(off)


def test_determinism_bitwise(orc):
    w = _workload("powerlaw", M=200_000)
    g = w.graph
    log(f"determinism: powerlaw M={g.M} nnz={g.nnz}")
    plan = make_plan(g)
    assert G.spmm_plan_info(plan)["n_heavy"] > 0
    _, _, _, Bd = to_dev(g, w.B)
    first = gpu_run(plan, g.M, Bd, "sum")[0]
    for _ in range(4):
        again = gpu_run(plan, g.M, Bd, "sum")[0]
        assert np.array_equal(first.view(np.uint32), again.view(np.uint32))
    fm, fa = gpu_run(plan, g.M, Bd, "max")
    for _ in range(2):
        m, a = gpu_run(plan, g.M, Bd, "max")
        assert np.array_equal(fm.view(np.uint32), m.view(np.uint32)) and np.array_equal(fa, a)
    G.spmm_plan_destroy(plan)


def test_descriptors_and_errors(orc):
    rng = np.random.default_rng(3)
    g = W.random_csr(rng, 5000, 4000, mean_deg=5.0, empty_frac=0.1, heavy_rows=3, heavy_deg=3000)
    plan = make_plan(g)
    info = G.spmm_plan_info(plan)
    d = orc.descriptors(g.rowptr, g.M)
    assert (info["M"], info["K"], info["nnz"]) == (g.M, g.K, d["nnz"])
    assert info["dmax"] == d["dmax"] and info["n_empty"] == d["n_empty"]
    assert abs(info["mean_deg"] - d["mean"]) <= 1e-12 * d["mean"]
    assert abs(info["cv_deg"] - d["cv"]) <= 1e-12 * d["cv"]
    G.spmm_plan_destroy(plan)

    # invalid CSR: the first bad row matches the oracle's validator
    rowptr = g.rowptr.copy()
    col = g.col.copy()
    bad_r = int(np.nonzero(g.degrees()[1234:] > 0)[0][0]) + 1234   # a non-empty row
    col[rowptr[bad_r]] = g.K + 5
    col[rowptr[bad_r + 700]] = -1
    assert orc.validate(rowptr, col, g.M, g.K) == bad_r
    rp, cl, vl, _ = to_dev(W.Graph("bad", g.M, g.K, rowptr, col, g.val))
    with pytest.raises(G.SpmmError) as ei:
        G.spmm_plan_create(rp, cl, vl, g.M, g.K)
    assert ei.value.status == G.SPMM_E_BAD_CSR and f"first bad row {bad_r}" in str(ei.value)
    rowptr2 = g.rowptr.copy()
    rowptr2[2001] = rowptr2[2002] + 1          # row 2001 gets a negative length
    bad2 = orc.validate(rowptr2, g.col, g.M, g.K)
    rp2 = torch.from_numpy(rowptr2).to(DEV)
    with pytest.raises(G.SpmmError) as ei:
        G.spmm_plan_create(rp2, cl, vl, g.M, g.K)
    assert ei.value.status == G.SPMM_E_BAD_CSR and f"first bad row {bad2}" in str(ei.value)

    # host memory where device memory is required
    host_rp = torch.from_numpy(g.rowptr)
    with pytest.raises(G.SpmmError) as ei:
        G.spmm_plan_create(host_rp, cl, vl, g.M, g.K)
    assert ei.value.status == G.SPMM_E_INVALID_ARG
    plan = make_plan(g)
    Bh = torch.zeros((g.K, 8), dtype=torch.float32)
    C = torch.empty((g.M, 8), dtype=torch.float32, device=DEV)
    with pytest.raises(ValueError):                      # the binding refuses a host tensor
        G.spmm_run(plan, Bh, C, None, 8, "sum")
    with pytest.raises(G.SpmmError) as ei:               # and so does the library, given its address
        G.spmm_run(plan, Bh.data_ptr(), C, None, 8, "sum")
    assert ei.value.status == G.SPMM_E_INVALID_ARG
    with pytest.raises(ValueError):                      # the binding refuses C [M, 8] as B [K, 8]
        G.spmm_run(plan, C, C, None, 8, "sum")
    with pytest.raises(G.SpmmError) as ei:               # the library refuses B overlapping C
        G.spmm_run(plan, C.data_ptr(), C, None, 8, "sum")
    assert ei.value.status == G.SPMM_E_INVALID_ARG and "overlaps" in str(ei.value)
    G.spmm_plan_destroy(plan)


def test_side_stream(orc):
    w = _workload("tiny")
    g = w.graph
    plan = make_plan(g)
    _, _, _, Bd = to_dev(g, w.B)
    s = torch.cuda.Stream()
    C = torch.empty((g.M, w.N), dtype=torch.float32, device=DEV)
    with torch.cuda.stream(s):
        G.spmm_run(plan, Bd, C, None, w.N, "mean", s)
    s.synchronize()
    check(orc, g, w.B, "mean", C.cpu().numpy(), None, exact_rows=np.arange(g.M), what="side stream")
    G.spmm_plan_destroy(plan)


MEDIUM = [("road", 60_000), ("powerlaw", 120_000), ("diffusion", 60_000), ("community", 12_000)]


@pytest.mark.parametrize("name,M", MEDIUM, ids=[m[0] for m in MEDIUM])
def test_regimes_medium_full_compare(orc, name, M):
    w = _workload(name, M=M)
    g = w.graph
    log(f"medium {name}: M={g.M} nnz={g.nnz} N={w.N}")
    plan = make_plan(g)
    light = G.spmm_plan_partition(plan)["light"]
    _, _, _, Bd = to_dev(g, w.B)
    for red in sorted(set(w.reduces) | {"max"}):
        C, arg = gpu_run(plan, g.M, Bd, red)
        check(orc, g, w.B, red, C, arg, exact_rows=light, what=f"{name} {red}")
    G.spmm_plan_destroy(plan)


FULL = ["road", "diffusion", "community", "powerlaw"]


@pytest.mark.parametrize("name", FULL)
def test_regimes_full_size_sampled(orc, name):
    """Full-size regimes in the benchmark's launch configuration (automatic
    routing), checked on a sample of rows: evenly spaced rows, the first and
    last rows, and the longest rows (all split rows for the power-law graph)."""
    w = _workload(name)
    g = w.graph
    log(f"full {name}: M={g.M} nnz={g.nnz} N={w.N}")
    plan = make_plan(g)
    info = G.spmm_plan_info(plan)
    part = G.spmm_plan_partition(plan)
    _, _, _, Bd = to_dev(g, w.B)
    deg = g.degrees()
    rng = np.random.default_rng(1)
    sample = np.unique(np.concatenate([
        np.arange(0, 64), np.arange(g.M - 64, g.M), rng.choice(g.M, size=3000, replace=False),
        np.argsort(deg)[-400:], np.unique(part["seg_row"])[:2000],
    ])).astype(np.int64)
    light_set = np.setdiff1d(sample, np.unique(part["seg_row"]), assume_unique=False)
    exact_idx = np.searchsorted(sample, light_set)
    log(f"  split: heavy={info['n_heavy']} pieces={info['n_seg']} sample={sample.size}")
    for red in w.reduces:
        C, arg = gpu_run(plan, g.M, Bd, red, poison=True)
        assert not np.isnan(C).any(), "unwritten output"
        check(orc, g, w.B, red, C[sample], None if arg is None else arg[sample], rows=sample,
              exact_rows=exact_idx, what=f"full {name} {red}")
    G.spmm_plan_destroy(plan)


@pytest.mark.parametrize("weighted,mode,K", [(False, 1, 15_000), (True, 1, 15_000), (False, 2, 15_000),
                                              (True, 1, 300_000)],
                         ids=["compact", "compact-weighted", "wide-forced", "wide-span"])
def test_row_tiles_match_csr_path(orc, weighted, mode, K):
    """Row-tile records (bounds + indexes in one record per 8 rows) give the same
    bits as the CSR path: compact 16-bit records, forced 32-bit records, and a
    graph whose column spans exceed 16 bits (the plan falls back to 32-bit
    records); tiles too long for a record take the CSR path inside the tile
    kernel, and the last tile is ragged."""
    rng = np.random.default_rng(404 + weighted + K)
    g = W.random_csr(rng, 20_003, K, mean_deg=3.0, empty_frac=0.05, heavy_rows=40, heavy_deg=150,
                     dup_frac=0.05, shuffle_rows=True, weighted=weighted)
    for N in (16, 64, 32):
        B = rng.standard_normal((g.K, N)).astype(np.float32)
        _, _, _, Bd = to_dev(g, B)
        on = make_plan(g, [(G.SPMM_OPT_TILES, mode)])
        off = make_plan(g, [(G.SPMM_OPT_TILES, 0)])
        info = G.spmm_plan_info(on)
        expect = 1 if (mode == 2 or K > 65536) else 2
        assert info["tiles"] == expect and info["tile_cap"] > 0, info["tiles"]
        assert info["tile_overflow"] >= 1            # the 150-entry rows overflow their tiles
        assert G.spmm_plan_info(off)["tiles"] == 0
        for red in ("sum", "mean", "max"):
            C1, a1 = gpu_run(on, g.M, Bd, red)
            assert G.spmm_plan_info(on)["route_tiled"] == 1, f"N={N}: tile kernel not routed"
            C0, a0 = gpu_run(off, g.M, Bd, red)
            assert G.spmm_plan_info(off)["route_tiled"] == 0
            log(f"tiles mode={mode} K={K} N={N} {red} cap={info['tile_cap']} kind={info['tiles']}")
            assert np.array_equal(C1.view(np.uint32), C0.view(np.uint32)), f"tiles vs CSR N={N} {red}"
            if a1 is not None:
                assert np.array_equal(a1, a0)
            check(orc, g, B, red, C1, a1, exact_rows=np.arange(g.M), what=f"tiles N={N} {red}")
        G.spmm_plan_destroy(on)
        G.spmm_plan_destroy(off)


def _sub_csr(g, M, K):
    """The first M rows of g, keeping only columns below K."""
    keep_rows = g.rowptr[: M + 1]
    cols = g.col[: keep_rows[-1]]
    vals = None if g.val is None else g.val[: keep_rows[-1]]
    rows = np.repeat(np.arange(M), np.diff(keep_rows))
    m = cols < K
    rowptr, col, order = W.csr_from_pairs(M, rows[m], cols[m])
    val = None if vals is None else vals[m][order]
    return W.Graph("sub", M, K, rowptr, col, val)


def _permute_within_rows(g, rng):
    """The same matrix with each row's entries (and values) in random order."""
    col = g.col.copy()
    val = None if g.val is None else g.val.copy()
    for i in range(g.M):
        a, b = g.rowptr[i], g.rowptr[i + 1]
        if b - a > 1:
            p = a + rng.permutation(b - a)
            col[a:b] = g.col[p]
            if val is not None:
                val[a:b] = g.val[p]
    return W.Graph(g.name, g.M, g.K, g.rowptr, col, val)


def _sort_within_rows(g):
    """The same matrix with each row's entries in column order (stable)."""
    rows = np.repeat(np.arange(g.M), np.diff(g.rowptr))
    order = np.lexsort((g.col, rows))
    return W.Graph(g.name, g.M, g.K, g.rowptr, g.col[order], None if g.val is None else g.val[order])


def test_window_forced_on_scattered_graph(orc):
    """The window forced on for a graph with few in-window entries: the sorted-row
    kernel's per-row run lengths are built by the option call, and the result is
    the row kernel's, bit for bit."""
    rng = np.random.default_rng(21)
    g = _sort_within_rows(W.random_csr(rng, 3_000, 2_000, mean_deg=9.0, empty_frac=0.05, dup_frac=0.05))
    B = rng.standard_normal((g.K, 136)).astype(np.float32)
    _, _, _, Bd = to_dev(g, B)
    on = make_plan(g, [(G.SPMM_OPT_WINDOW, 1)])
    off = make_plan(g, [(G.SPMM_OPT_WINDOW, 0)])
    assert G.spmm_plan_info(on)["win_frac"] < 0.5
    for red in ("sum", "mean", "max"):
        C1, a1 = gpu_run(on, g.M, Bd, red)
        assert G.spmm_plan_info(on)["route_window"] == 2
        C0, a0 = gpu_run(off, g.M, Bd, red)
        assert np.array_equal(C1.view(np.uint32), C0.view(np.uint32)), red
        if a1 is not None:
            assert np.array_equal(a1, a0)
        check(orc, g, B, red, C1, a1, exact_rows=np.arange(g.M), what=f"forced window {red}")
    G.spmm_plan_destroy(on)
    G.spmm_plan_destroy(off)


@pytest.mark.parametrize("order", ["sorted", "shuffled"])
@pytest.mark.parametrize("shape", ["square", "wide", "tall", "unweighted", "duplicates", "long rows"])
def test_community_window_matches_row_kernel(orc, shape, order):
    """Both LDS window kernels (B's 256-row blocks staged per workgroup) give
    the row kernel's bits, with a ragged last block, N not a multiple of the
    64-column slice, K different from M, repeated columns and rows longer
    than a staging chunk: rows in column order take the three-run kernel
    (route 2), others the per-entry kernel (route 1)."""
    g = W.make_graph("community", M=5_000, seed=11)
    if shape == "wide":
        g = _sub_csr(g, 4_000, 5_000)
    elif shape == "tall":
        g = _sub_csr(g, 5_000, 4_100)
    elif shape == "unweighted":
        g = W.Graph("u", g.M, g.K, g.rowptr, g.col, None)
    elif shape == "duplicates":
        g = W.block_csr(np.random.default_rng(5), 3_000, 3_000, in_deg=40.0, off_deg=3.0)
    elif shape == "long rows":      # rows of ~240 entries: runs cross the 128-entry staging chunks
        g = W.block_csr(np.random.default_rng(6), 1_500, 1_600, in_deg=180.0, off_deg=60.0)
    rng = np.random.default_rng(77)
    g = _sort_within_rows(g) if order == "sorted" else _permute_within_rows(g, rng)
    want_route = 2 if order == "sorted" else 1
    for N in (128, 200, 512):
        B = rng.standard_normal((g.K, N)).astype(np.float32)
        _, _, _, Bd = to_dev(g, B)
        on = make_plan(g, [(G.SPMM_OPT_WINDOW, 1)])
        off = make_plan(g, [(G.SPMM_OPT_WINDOW, 0)])
        assert G.spmm_plan_info(on)["win_frac"] > 0.5
        for red in ("sum", "mean", "max"):
            C1, a1 = gpu_run(on, g.M, Bd, red)
            assert G.spmm_plan_info(on)["route_window"] == want_route
            C0, a0 = gpu_run(off, g.M, Bd, red)
            assert G.spmm_plan_info(off)["route_window"] == 0
            log(f"window {shape} N={N} {red}")
            assert np.array_equal(C1.view(np.uint32), C0.view(np.uint32)), f"window vs row kernel {shape} N={N} {red}"
            if a1 is not None:
                assert np.array_equal(a1, a0)
            check(orc, g, B, red, C1, a1, exact_rows=np.arange(g.M), what=f"window {shape} N={N} {red}")
        G.spmm_plan_destroy(on)
        G.spmm_plan_destroy(off)


def test_router_rules():
    """Routing decisions measured on the GPU (the router sweep): community
    structure takes the LDS window kernel from 64 columns; launch-bound small
    graphs take float1 lanes below 128 columns, 8 lanes per row up to 32
    vectors, and no coarsening; skewed
    graphs take 64-column slices from 128 columns, 128-column slices from 256
    to 512 and 64-column slices above; widths of a multiple of 8 vectors that
    are not powers of two (96, 160, 192 floats) take 8 lanes x 2 vectors at
    low degree and half the lanes coarsened otherwise; wide features at
    higher degree take 64 lanes without coarsening; V = 2 panels take the
    largest power-of-two factor of a width that is not a power of two as
    their lane count, and community-structured graphs take the window kernel
    instead of panels for such widths above 256 floats."""
    community = make_plan(W.make_graph("community", M=20_000))
    for N, win in ((16, 0), (64, 2), (128, 2), (512, 2)):
        info = G.spmm_plan_route(community, N, "sum")
        assert (info["route_window"] > 0) == (win > 0), (N, info["route_window"])
    G.spmm_plan_destroy(community)
    tiny = make_plan(W.make_graph("tiny"))
    for N, vec, lanes in ((16, 1, 8), (64, 1, 64), (128, 4, 8), (512, 4, 64)):
        info = G.spmm_plan_route(tiny, N, "sum")
        assert (info["route_vec"], info["route_lanes"], info["route_coarsen"]) == (vec, lanes, 1), (N, info)
    G.spmm_plan_destroy(tiny)
    rng = np.random.default_rng(5)
    skew = make_plan(W.random_csr(rng, 20_000, 20_000, mean_deg=6.0, heavy_rows=20, heavy_deg=5000))
    assert G.spmm_plan_info(skew)["cv_deg"] > 1.0
    for N, lanes in ((96, 32), (128, 16), (192, 16), (256, 32), (512, 32), (1024, 16)):
        info = G.spmm_plan_route(skew, N, "sum")
        assert (info["route_lanes"], info["route_coarsen"]) == (lanes, 1), (N, info)
    G.spmm_plan_destroy(skew)
    road = make_plan(W.make_graph("road", M=100_000))
    for N, lg in ((64, (8, 2)), (96, (8, 2)), (100, (16, 2)), (160, (8, 2)), (192, (8, 2))):
        info = G.spmm_plan_route(road, N, "sum")
        assert (info["route_lanes"], info["route_coarsen"]) == lg, (N, info)
    G.spmm_plan_destroy(road)
    diffusion = make_plan(W.make_graph("diffusion", M=100_000))
    for N, lg in ((96, (16, 2)), (100, (32, 1)), (160, (32, 2)), (192, (32, 2)), (300, (64, 2)),
                  (512, (64, 1)), (1024, (64, 1))):
        info = G.spmm_plan_route(diffusion, N, "mean")
        assert (info["route_lanes"], info["route_coarsen"]) == lg, (N, info)
    G.spmm_plan_destroy(diffusion)
    knn = make_plan(W.knn_line(50_000, 10))
    assert G.spmm_plan_info(knn)["pairs_built"] == 1
    for N, panels, lanes in ((96, 1, 8), (100, 1, 32), (128, 1, 32), (160, 1, 8), (192, 1, 16), (256, 1, 32),
                             (300, 0, 16), (512, 0, 16)):
        info = G.spmm_plan_route(knn, N, "sum")
        assert info["route_pairs"] == panels and (panels or info["route_window"] > 0), (N, info)
        assert info["route_lanes"] == lanes, (N, info)
    G.spmm_plan_destroy(knn)

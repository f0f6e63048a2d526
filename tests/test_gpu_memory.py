"""Device-memory limits through the C ABI: every call that allocates, run with
a limit below what it needs, must fail with SPMM_E_OOM naming the buffer,
free what it allocated, and leave the plan usable; with the limit at its
measured need it must succeed.

The pages say nothing about memory limits; the contract tested here is the
library's own (the header's "Device memory" section): a per-thread limit on
what one call may hold (spmm_set_mem_limit) and a per-plan limit
(SPMM_OPT_MEM_LIMIT).  Plan generations (bumped when an option replaces
device buffers) are checked here too.
"""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gnn_sparse_dense_amd as G
    from tests.gpu_helpers import DEV, check, gpu_run, log, make_plan, to_dev


def _in_use():
    return G.spmm_mem_stats()["in_use"]


def _limits(peak):
    return sorted({peak - 1, peak * 3 // 4, peak // 2, peak // 8, 1})


def _sweep(name, call, cleanup, after_failure=None):
    """Measure the call's peak, then require OOM (and no leak) at limits
    below it and success at it."""
    G.spmm_set_mem_limit(0)
    base = _in_use()
    out = call()
    st = G.spmm_mem_stats()
    peak, nalloc = st["last_call_peak"], st["last_call_allocs"]
    log(f"{name}: peak {peak} bytes in {nalloc} allocations")
    assert peak > 0 and nalloc > 0, name
    cleanup(out)
    assert _in_use() == base, f"{name}: memory not returned after cleanup"
    for L in _limits(peak):
        G.spmm_set_mem_limit(L)
        try:
            with pytest.raises(G.SpmmError) as ei:
                call()
        finally:
            G.spmm_set_mem_limit(0)
        msg = str(ei.value)
        assert ei.value.status == G.SPMM_E_OOM, f"{name} at limit {L}: {msg}"
        assert "exceeds the memory limit" in msg and f"limit of {L} bytes" in msg, msg
        assert _in_use() == base, f"{name} at limit {L}: {_in_use() - base} bytes left behind"
        if after_failure is not None:
            after_failure()
    G.spmm_set_mem_limit(peak)
    try:
        out = call()
    finally:
        G.spmm_set_mem_limit(0)
    cleanup(out)
    assert _in_use() == base


def _product_ok(orc, plan, g, B, Bd):
    for red in ("sum", "max"):
        C, arg = gpu_run(plan, g.M, Bd, red)
        check(orc, g, B, red, C, arg, what=f"after a failed build ({red})")


def _skewed():
    rng = np.random.default_rng(31)
    return W.random_csr(rng, 3000, 2500, mean_deg=6.0, empty_frac=0.05, heavy_rows=3, heavy_deg=3000)


def test_plan_create_and_graph_calls_under_limits(orc):
    rng = np.random.default_rng(5)
    g = _skewed()
    rowptr, col, val, _ = to_dev(g)
    _sweep("plan create", lambda: G.spmm_plan_create(rowptr, col, val, g.M, g.K), G.spmm_plan_destroy)

    plan = make_plan(g)
    B = rng.standard_normal((g.K, 16)).astype(np.float32)
    _, _, _, Bd = to_dev(g, B)
    after = lambda: _product_ok(orc, plan, g, B, Bd)  # noqa: E731
    _sweep("transpose", lambda: G.spmm_plan_transpose(plan, 1), G.spmm_plan_destroy, after)
    _sweep("features", lambda: G.spmm_plan_features(plan, 2), lambda out: None, after)
    G.spmm_plan_destroy(plan)

    # square graphs: reordering and permuting
    sq = W.random_csr(rng, 2000, 2000, mean_deg=5.0, empty_frac=0.05)
    plan = make_plan(sq)
    Bs = rng.standard_normal((sq.K, 8)).astype(np.float32)
    _, _, _, Bsd = to_dev(sq, Bs)
    after = lambda: _product_ok(orc, plan, sq, Bs, Bsd)  # noqa: E731
    _sweep("reorder", lambda: G.spmm_plan_reorder(plan), lambda out: None, after)
    perm = torch.from_numpy(rng.permutation(sq.M).astype(np.int64)).to(DEV)
    _sweep("permute", lambda: G.spmm_plan_permute(plan, perm), G.spmm_plan_destroy, after)
    G.spmm_plan_destroy(plan)

    # edge list -> CSR
    E = 20000
    row = torch.from_numpy(rng.integers(0, 3000, E).astype(np.int64)).to(DEV)
    cl = torch.from_numpy(rng.integers(0, 2000, E).astype(np.int64)).to(DEV)
    vl = torch.from_numpy(rng.random(E, dtype=np.float32)).to(DEV)
    _sweep("edge list to CSR", lambda: G.spmm_coo_to_csr(row, cl, vl, 3000, 2000), lambda out: None)


OPTION_CASES = [
    # (name, graph maker, option, value, options set first)
    ("row split", "skewed", "SPMM_OPT_SPLIT_MODE", 1, [("SPMM_OPT_SPLIT_MODE", 0)]),
    ("row tiles", "uniform", "SPMM_OPT_TILES", 1, [("SPMM_OPT_TILES", 0)]),
    ("window runs", "block", "SPMM_OPT_WINDOW", 1, []),
    ("fp16 tiles", "community", "SPMM_OPT_MFMA", 1, []),
    ("split fp16 tiles", "community", "SPMM_OPT_MFMA", 2, []),
    ("V = 2 panels", "knn", "SPMM_OPT_VBLOCK", 2, [("SPMM_OPT_VBLOCK", 0)]),
    ("automatic V = 2 panels", "knn", "SPMM_OPT_VBLOCK", -1, [("SPMM_OPT_VBLOCK", 0)]),
    ("merge path", "skewed", "SPMM_OPT_BALANCE", 1, []),
]


def _graph(kind):
    rng = np.random.default_rng(77)
    if kind == "skewed":
        return _skewed()
    if kind == "uniform":
        return W.random_csr(rng, 4000, 4000, mean_deg=4.0, empty_frac=0.05)
    if kind == "block":
        # sorted rows, less than half the entries inside their block: no window
        # runs are built at plan creation
        g = W.block_csr(rng, 3000, 3000, in_deg=4.0, off_deg=8.0)
        for i in range(g.M):
            a, b = g.rowptr[i], g.rowptr[i + 1]
            g.col[a:b] = np.sort(g.col[a:b])
        return g
    if kind == "community":
        return W.make_graph("community", M=3000)
    if kind == "knn":
        return W.knn_line(3000, 10)
    raise ValueError(kind)


@pytest.mark.parametrize("name,kind,opt,value,pre", OPTION_CASES, ids=[c[0] for c in OPTION_CASES])
def test_option_builds_under_limits(orc, name, kind, opt, value, pre):
    rng = np.random.default_rng(9)
    g = _graph(kind)
    plan = make_plan(g, [(getattr(G, o), v) for o, v in pre])
    N = 64
    B = rng.standard_normal((g.K, N)).astype(np.float32)
    _, _, _, Bd = to_dev(g, B)
    o = getattr(G, opt)
    off = {"SPMM_OPT_SPLIT_MODE": 0, "SPMM_OPT_TILES": 0, "SPMM_OPT_WINDOW": 0,
           "SPMM_OPT_MFMA": 0, "SPMM_OPT_VBLOCK": 0, "SPMM_OPT_BALANCE": 0}[opt]

    if kind == "block":
        assert G.spmm_plan_info(plan)["win_frac"] < 0.5      # no runs built at creation

    def after():
        _product_ok(orc, plan, g, B, Bd)

    _sweep(name, lambda: G.spmm_plan_set_option(plan, o, value), lambda out: G.spmm_plan_set_option(plan, o, off),
           after)
    G.spmm_plan_destroy(plan)


def test_failed_split_rebuild_keeps_the_previous_split(orc):
    """A split rebuild that does not fit the plan's limit puts the previous
    split back (same partition, same bits)."""
    rng = np.random.default_rng(14)
    g = _skewed()
    plan = make_plan(g)
    info = G.spmm_plan_info(plan)
    assert info["n_seg"] > 0
    B = rng.standard_normal((g.K, 64)).astype(np.float32)
    _, _, _, Bd = to_dev(g, B)
    before = gpu_run(plan, g.M, Bd, "sum")[0]
    part = G.spmm_plan_partition(plan)
    G.spmm_plan_set_option(plan, G.SPMM_OPT_MEM_LIMIT, info["device_bytes"])
    with pytest.raises(G.SpmmError) as ei:
        G.spmm_plan_set_option(plan, G.SPMM_OPT_SPLIT_L, 128)       # 4x the pieces
    assert ei.value.status == G.SPMM_E_OOM
    after = G.spmm_plan_info(plan)
    assert (after["n_seg"], after["split_L"], after["device_bytes"]) == (info["n_seg"], info["split_L"],
                                                                         info["device_bytes"])
    part2 = G.spmm_plan_partition(plan)
    for k in ("seg_row", "seg_begin", "seg_end", "light"):
        assert np.array_equal(part[k], part2[k]), k
    again = gpu_run(plan, g.M, Bd, "sum")[0]
    assert np.array_equal(before.view(np.uint32), again.view(np.uint32))
    check(orc, g, B, "sum", again, None, what="restored split")
    G.spmm_plan_set_option(plan, G.SPMM_OPT_MEM_LIMIT, 0)
    G.spmm_plan_set_option(plan, G.SPMM_OPT_SPLIT_L, 128)
    assert G.spmm_plan_info(plan)["n_seg"] > info["n_seg"]
    G.spmm_plan_destroy(plan)


def test_plan_limit_and_generation(orc):
    rng = np.random.default_rng(12)
    g = W.make_graph("community", M=3000)
    plan = make_plan(g)
    B = rng.standard_normal((g.K, 64)).astype(np.float32)
    _, _, _, Bd = to_dev(g, B)
    info = G.spmm_plan_info(plan)
    held, gen0 = info["device_bytes"], info["generation"]
    assert held > 0 and info["mem_limit"] == 0
    G.spmm_plan_set_option(plan, G.SPMM_OPT_MEM_LIMIT, held + 1)
    assert G.spmm_plan_info(plan)["mem_limit"] == held + 1
    base = _in_use()
    for opt, v in ((G.SPMM_OPT_MFMA, 1), (G.SPMM_OPT_VBLOCK, 1), (G.SPMM_OPT_BALANCE, 1)):
        with pytest.raises(G.SpmmError) as ei:
            G.spmm_plan_set_option(plan, opt, v)
        assert ei.value.status == G.SPMM_E_OOM and f"limit of {held + 1} bytes" in str(ei.value)
        assert _in_use() == base
    with pytest.raises(G.SpmmError) as ei:
        G.spmm_plan_transpose(plan, 0)
    assert ei.value.status == G.SPMM_E_OOM
    assert _in_use() == base
    _product_ok(orc, plan, g, B, Bd)
    assert G.spmm_plan_info(plan)["generation"] == gen0     # nothing was replaced
    # options that only steer the router keep the generation
    G.spmm_plan_set_option(plan, G.SPMM_OPT_MEM_LIMIT, 0)
    G.spmm_plan_set_option(plan, G.SPMM_OPT_LANES, 8)
    G.spmm_plan_set_option(plan, G.SPMM_OPT_LANES, 0)
    assert G.spmm_plan_info(plan)["generation"] == gen0
    # building, re-setting and freeing a structure
    G.spmm_plan_set_option(plan, G.SPMM_OPT_MFMA, 1)
    assert G.spmm_plan_info(plan)["generation"] == gen0 + 1
    G.spmm_plan_set_option(plan, G.SPMM_OPT_MFMA, 1)         # already built: unchanged
    assert G.spmm_plan_info(plan)["generation"] == gen0 + 1
    G.spmm_plan_set_option(plan, G.SPMM_OPT_MFMA, 0)
    assert G.spmm_plan_info(plan)["generation"] == gen0 + 2
    assert G.spmm_plan_info(plan)["device_bytes"] == held
    G.spmm_plan_destroy(plan)
    with pytest.raises(G.SpmmError):
        G.spmm_set_mem_limit(-1)

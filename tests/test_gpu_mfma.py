"""GPU parity of the fp16 matrix-core tile path (option SPMM_OPT_MFMA) through
the C ABI.

Contract of that path: |GPU - oracle| <= 2e-3 * sum_p |a_p * b_p| + 1e-4 per
element for sum and mean (fp16 operands, fp32 accumulation), bitwise
reproducible runs; max runs, widths that are not a multiple of 4 and the
option switched off keep the fp32 kernels and their exact contract.

Besides the oracle gate, `test_tile_rounding_model` compares with a float64
model of the path's own roundings (in-block weights summed in fp32 and rounded
to fp16, B rounded to fp16, residual entries in fp32) at fp32-accumulation
tolerance: a misplaced fragment or a lost entry shows there as an O(1) error
even where the fp16 contract would absorb it.
"""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gnn_sparse_dense_amd as G
    from tests.gpu_helpers import DEV, check, gpu_run, log, make_plan, to_dev

TILE_REL = 2e-3
TILE_ABS = 1e-4


def check_tiles(orc, g, B, reduce, C, rows=None, what=""):
    ref = orc.spmm(g.rowptr, g.col, g.val, g.M, g.K, B, reduce, rows=rows)
    S = orc.sumabs(g.rowptr, g.col, g.val, g.M, B, rows=rows)
    err = np.abs(C.astype(np.float64) - ref.astype(np.float64))
    bad = ~(err <= TILE_REL * S + TILE_ABS)
    log(f"{what}: max err {np.nanmax(err):.3e}, max err/S {np.nanmax(err / np.maximum(S, 1e-30)):.3e}")
    assert not bad.any(), f"{what}: {int(bad.sum())} of {bad.size} outside the fp16 tile tolerance"


def tile_plan(g):
    plan = make_plan(g)
    G.spmm_plan_set_option(plan, G.SPMM_OPT_MFMA, 1)
    return plan


CASES = [
    ("community", dict(M=6000), 512),
    ("community", dict(M=6000), 64),
    ("community", dict(M=6000), 68),      # partial last column slice
    ("community", dict(M=6000), 4),
    ("block", dict(M=1500, K=700), 64),   # rows beyond K: blocks without columns
    ("block", dict(M=700, K=1500), 132),
    ("block_unweighted", dict(M=1000, K=1000), 128),
]


def _graph(name, kw, seed):
    if name == "community":
        return W.make_graph("community", M=kw["M"])
    rng = np.random.default_rng(seed)
    return W.block_csr(rng, kw["M"], kw["K"], weighted=(name == "block"))


@pytest.mark.parametrize("name,kw,N", CASES, ids=[f"{c[0]}-{c[2]}" for c in CASES])
@pytest.mark.parametrize("reduce", ["sum", "mean"])
def test_tile_parity(orc, name, kw, N, reduce):
    g = _graph(name, kw, seed=N)
    rng = np.random.default_rng(100 + N)
    B = rng.standard_normal((g.K, N)).astype(np.float32)
    log(f"tiles {name} M={g.M} K={g.K} nnz={g.nnz} N={N} {reduce}")
    plan = tile_plan(g)
    _, _, _, Bd = to_dev(g, B)
    C, _ = gpu_run(plan, g.M, Bd, reduce)
    info = G.spmm_plan_info(plan)
    assert info["mfma_tiles"] == 1 and info["route_mfma"] == 1
    r = np.repeat(np.arange(g.M), np.diff(g.rowptr))
    assert info["mfma_resid_nnz"] == int(((g.col // 256) != (r // 256)).sum())
    check_tiles(orc, g, B, reduce, C, what=f"{name} N={N} {reduce}")
    C2, _ = gpu_run(plan, g.M, Bd, reduce)
    assert np.array_equal(C.view(np.uint32), C2.view(np.uint32)), "runs differ"
    G.spmm_plan_destroy(plan)


def _rounding_model(g, B):
    """float64 model of the tile path: per row, the in-block weights of each
    column summed in fp32 in stored order and rounded to fp16, times B rounded
    to fp16; the other entries in fp32 as stored.  Returns (C, sum of |terms|)."""
    M, N = g.M, B.shape[1]
    B16 = B.astype(np.float16).astype(np.float64)
    B64 = B.astype(np.float64)
    C = np.zeros((M, N))
    S = np.zeros((M, N))
    for i in range(M):
        a, b = g.rowptr[i], g.rowptr[i + 1]
        w0 = (i // 256) * 256
        sums = {}
        for p in range(a, b):
            c = int(g.col[p])
            w = np.float32(1.0) if g.val is None else g.val[p]
            if w0 <= c < w0 + 256:
                sums[c] = np.float32(sums.get(c, np.float32(0.0)) + w)
            else:
                C[i] += np.float64(w) * B64[c]
                S[i] += abs(np.float64(w) * B64[c])
        for c, w in sums.items():
            w16 = np.float64(np.float16(w))
            C[i] += w16 * B16[c]
            S[i] += np.abs(w16 * B16[c])
    return C, S


@pytest.mark.parametrize("weighted", [True, False])
def test_tile_rounding_model(orc, weighted):
    rng = np.random.default_rng(7)
    g = W.block_csr(rng, 900, 800, in_deg=20.0, off_deg=3.0, weighted=weighted)
    B = rng.standard_normal((g.K, 72)).astype(np.float32)
    B = np.where(np.abs(B) < 1e-3, np.copysign(1e-3, B), B).astype(np.float32)   # no fp16 subnormals
    plan = tile_plan(g)
    _, _, _, Bd = to_dev(g, B)
    C, _ = gpu_run(plan, g.M, Bd, "sum")
    ref, S = _rounding_model(g, B)
    err = np.abs(C - ref)
    log(f"rounding model weighted={weighted}: max err {err.max():.3e}")
    assert (err <= 2e-5 * S + 1e-6).all(), f"{int((err > 2e-5 * S + 1e-6).sum())} elements off the model"
    G.spmm_plan_destroy(plan)


def test_tile_fallbacks_and_option(orc):
    rng = np.random.default_rng(3)
    g = W.block_csr(rng, 1200, 1200)
    plan = tile_plan(g)
    B = rng.integers(0, 4, size=(g.K, 16)).astype(np.float32)
    _, _, _, Bd = to_dev(g, B)
    # max keeps the fp32 kernels: bit-exact with the oracle
    C, arg = gpu_run(plan, g.M, Bd, "max")
    assert G.spmm_plan_info(plan)["route_mfma"] == 0
    check(orc, g, B, "max", C, arg, what="max with tiles enabled")
    # N not a multiple of 4 keeps the fp32 kernels
    B6 = rng.standard_normal((g.K, 6)).astype(np.float32)
    _, _, _, B6d = to_dev(g, B6)
    C, _ = gpu_run(plan, g.M, B6d, "sum")
    assert G.spmm_plan_info(plan)["route_mfma"] == 0
    check(orc, g, B6, "sum", C, None, what="N=6 with tiles enabled")
    # switching the option off frees the tiles and restores the fp32 route
    G.spmm_plan_set_option(plan, G.SPMM_OPT_MFMA, 0)
    info = G.spmm_plan_info(plan)
    assert info["mfma_tiles"] == 0 and info["mfma_resid_nnz"] == 0
    C, _ = gpu_run(plan, g.M, Bd, "sum")
    assert G.spmm_plan_info(plan)["route_mfma"] == 0
    check(orc, g, B, "sum", C, None, what="tiles off")
    with pytest.raises(G.SpmmError) as ei:
        G.spmm_plan_set_option(plan, G.SPMM_OPT_MFMA, 3)
    assert ei.value.status == G.SPMM_E_INVALID_ARG
    G.spmm_plan_destroy(plan)


def test_tile_range_refused(orc):
    rng = np.random.default_rng(4)
    g = W.block_csr(rng, 300, 300)
    g.val[:] = 70000.0                     # in-block weights beyond fp16
    plan = make_plan(g)
    with pytest.raises(G.SpmmError) as ei:
        G.spmm_plan_set_option(plan, G.SPMM_OPT_MFMA, 1)
    assert ei.value.status == G.SPMM_E_UNSUPPORTED
    assert G.spmm_plan_info(plan)["mfma_tiles"] == 0
    G.spmm_plan_destroy(plan)


def test_tile_full_community_sampled(orc):
    w = W.make("community")
    g, B = w.graph, w.B
    log(f"full community M={g.M} nnz={g.nnz} N={B.shape[1]}")
    plan = tile_plan(g)
    _, _, _, Bd = to_dev(g, B)
    C, _ = gpu_run(plan, g.M, Bd, "sum")
    assert G.spmm_plan_info(plan)["route_mfma"] == 1
    rows = np.unique(np.concatenate([np.linspace(0, g.M - 1, 400).astype(np.int64),
                                     np.arange(g.M - 40, g.M), np.arange(0, 300)]))
    check_tiles(orc, g, B, "sum", C[rows], rows=rows, what="full community (sampled rows)")
    G.spmm_plan_destroy(plan)


# ---- split tiles (SPMM_OPT_MFMA = 2): the fp32 contract ----

def split_plan(g):
    plan = make_plan(g)
    G.spmm_plan_set_option(plan, G.SPMM_OPT_MFMA, 2)
    assert G.spmm_plan_info(plan)["mfma_tiles"] == 2
    return plan


SPLIT_CASES = [
    ("community", dict(M=6000), 512),
    ("community", dict(M=6000), 68),
    ("block", dict(M=1500, K=700), 64),
    ("block_unweighted", dict(M=1000, K=1000), 128),
]


@pytest.mark.parametrize("name,kw,N", SPLIT_CASES, ids=[f"{c[0]}-{c[2]}" for c in SPLIT_CASES])
@pytest.mark.parametrize("reduce", ["sum", "mean"])
def test_split_tiles_fp32_contract(orc, name, kw, N, reduce):
    g = _graph(name, kw, seed=N + 1)
    rng = np.random.default_rng(300 + N)
    B = rng.standard_normal((g.K, N)).astype(np.float32)
    plan = split_plan(g)
    _, _, _, Bd = to_dev(g, B)
    C, _ = gpu_run(plan, g.M, Bd, reduce)
    assert G.spmm_plan_info(plan)["route_mfma"] == 1
    check(orc, g, B, reduce, C, None, what=f"split {name} N={N} {reduce}")
    C2, _ = gpu_run(plan, g.M, Bd, reduce)
    assert np.array_equal(C.view(np.uint32), C2.view(np.uint32)), "runs differ"
    G.spmm_plan_destroy(plan)


def test_split_tiles_wide_range(orc):
    rng = np.random.default_rng(31)
    g = W.block_csr(rng, 2048, 2048, in_deg=20.0, off_deg=3.0)
    rows = np.repeat(np.arange(g.M), g.degrees())
    scale = np.float32(10.0) ** ((rows // 256) % 7 - 3).astype(np.float32)   # 1e-3 .. 1e3 by block
    g.val = (g.val * scale).astype(np.float32)
    B = rng.standard_normal((g.K, 64)).astype(np.float32)
    B[:, :32] *= np.float32(1e4)
    B[rng.random(B.shape) < 0.05] *= np.float32(1e-6)
    plan = split_plan(g)
    _, _, _, Bd = to_dev(g, B)
    for red in ("sum", "mean"):
        C, _ = gpu_run(plan, g.M, Bd, red)
        check(orc, g, B, red, C, None, what=f"split wide range {red}")
    # mode changes rebuild or free the tiles
    G.spmm_plan_set_option(plan, G.SPMM_OPT_MFMA, 1)
    assert G.spmm_plan_info(plan)["mfma_tiles"] == 1
    G.spmm_plan_set_option(plan, G.SPMM_OPT_MFMA, 2)
    assert G.spmm_plan_info(plan)["mfma_tiles"] == 2
    G.spmm_plan_set_option(plan, G.SPMM_OPT_MFMA, 0)
    assert G.spmm_plan_info(plan)["mfma_tiles"] == 0
    G.spmm_plan_destroy(plan)


def test_split_tiles_full_community_sampled(orc):
    w = W.make("community")
    g, B = w.graph, w.B
    plan = split_plan(g)
    _, _, _, Bd = to_dev(g, B)
    C, _ = gpu_run(plan, g.M, Bd, "sum")
    rows = np.unique(np.concatenate([np.linspace(0, g.M - 1, 400).astype(np.int64),
                                     np.arange(g.M - 40, g.M), np.arange(0, 300)]))
    check(orc, g, B, "sum", C[rows], None, rows=rows, what="split full community (sampled rows)")
    G.spmm_plan_destroy(plan)

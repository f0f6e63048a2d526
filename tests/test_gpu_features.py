"""GPU parity of spmm_plan_features (ParamSpMM Table 3 features) against the
oracle, through the C ABI: integer features exact, ratios within 1e-12
(relative)."""
import os

import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gnn_sparse_dense_amd as G
    from tests.gpu_helpers import log, make_plan

INTS = ("n", "n_nonempty", "nnz", "dmax", "max_bandwidth", "nnz_distinct", "nnz_vectors")
REALS = ("delta", "mean_deg", "mean_deg_nonempty", "cv_deg", "cv_deg_nonempty", "density", "mean_bandwidth",
         "padding_ratio")


def compare(orc, g, V, what):
    plan = make_plan(g)
    got = G.spmm_plan_features(plan, V)
    ref = orc.features(g.rowptr, g.col, g.M, g.K, V)
    log(f"{what} V={V}: padding {got['padding_ratio']:.4f} bandwidth {got['mean_bandwidth']:.1f}")
    for k in INTS:
        assert got[k] == ref[k], (what, V, k, got[k], ref[k])
    for k in REALS:
        assert abs(got[k] - ref[k]) <= 1e-12 * max(1.0, abs(ref[k])), (what, V, k, got[k], ref[k])
    assert got["V"] == V
    info = G.spmm_plan_info(plan)
    assert got["win_frac"] == info["win_frac"] and got["split_ratio"] == info["split_ratio"]
    G.spmm_plan_destroy(plan)


def test_features_golden(orc):
    kv = {}
    for line in open(os.path.join(os.path.dirname(__file__), "golden", "features_hand.txt")):
        if line.strip() and not line.startswith("#"):
            k, *v = line.split()
            kv[k] = v
    g = W.Graph("golden", int(kv["M"][0]), int(kv["K"][0]), np.array(kv["rowptr"], np.int64),
                np.array(kv["col"], np.int64), None)
    for V in (1, 2, 3):
        compare(orc, g, V, "golden")


@pytest.mark.parametrize("V", [1, 2, 3, 4, 64])
def test_features_irregular(orc, V):
    rng = np.random.default_rng(200 + V)
    g = W.random_csr(rng, 7001, 5003, mean_deg=9.0, empty_frac=0.2, dup_frac=0.3, shuffle_rows=True,
                     heavy_rows=3, heavy_deg=4000)
    compare(orc, g, V, "irregular")


@pytest.mark.parametrize("name,M", [("road", 50_000), ("powerlaw", 60_000), ("community", 20_000),
                                    ("diffusion", 50_000), ("tiny", None)])
def test_features_regimes(orc, name, M):
    compare(orc, W.make_graph(name, M=M), 2, name)


@pytest.mark.parametrize("name", ["road", "diffusion"])
def test_features_full_size(orc, name):
    compare(orc, W.make_graph(name), 2, name + " full")


def test_features_degenerate_and_errors(orc):
    empty = W.Graph("empty", 5, 4, np.zeros(6, np.int64), np.zeros(0, np.int64), None)
    compare(orc, empty, 2, "no entries")
    plan = make_plan(empty)
    for bad in (0, 65):
        with pytest.raises(G.SpmmError) as ei:
            G.spmm_plan_features(plan, bad)
        assert ei.value.status == G.SPMM_E_INVALID_ARG
    G.spmm_plan_destroy(plan)

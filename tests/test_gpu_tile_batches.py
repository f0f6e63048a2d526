"""GPU: 4-lane float4 row tiles at mean degree 8 and above take their entries
in batches of 4 instead of 8 (sum and mean).  Same fold order, so the bits
must equal the CSR row kernel's and the oracle's fused mode on every row;
graphs of exactly 10 entries per row (the diffusion recipe), and near-regular
weighted graphs with empty rows and a few long rows whose tiles overflow to
the CSR path inside the tile kernel, in compact and 32-bit records."""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gnn_sparse_dense_amd as G
    from tests.gpu_helpers import check, gpu_run, log, make_plan, to_dev


def _graphs():
    rng = np.random.default_rng(8_100)
    yield "diffusion", W.make_graph("diffusion", M=30_000)
    yield "near-regular", W.random_csr(rng, 20_011, 20_011, mean_deg=12.0, empty_frac=0.03, heavy_rows=12,
                                       heavy_deg=120, shuffle_rows=True, weighted=True)


@pytest.mark.parametrize("tiles", [1, 2])
def test_tile_batches_of_four(orc, tiles):
    for name, g in _graphs():
        assert g.nnz / g.M >= 8.0
        rng = np.random.default_rng(8_200 + tiles)
        for N in (16, 8, 13):
            B = rng.standard_normal((g.K, N)).astype(np.float32)
            _, _, _, Bd = to_dev(g, B)
            on = make_plan(g, [(G.SPMM_OPT_TILES, tiles)])
            off = make_plan(g, [(G.SPMM_OPT_TILES, 0)])
            for red in ("sum", "mean", "max"):
                C1, a1 = gpu_run(on, g.M, Bd, red)
                info = G.spmm_plan_info(on)
                route = (info["route_tiled"], info["route_lanes"], info["route_vec"], info["route_coarsen"])
                log(f"tile batches {name} tiles={tiles} N={N} {red} route={route} "
                    f"overflow={info['tile_overflow']}")
                assert route == (1, 4, 4, 1), f"{name} N={N}: {route}"
                C0, a0 = gpu_run(off, g.M, Bd, red)
                assert G.spmm_plan_info(off)["route_tiled"] == 0
                assert np.array_equal(C1.view(np.uint32), C0.view(np.uint32)), f"{name} N={N} {red}"
                if a1 is not None:
                    assert np.array_equal(a1, a0)
                check(orc, g, B, red, C1, a1, exact_rows=np.arange(g.M), what=f"{name} N={N} {red}")
            if name == "near-regular":
                assert G.spmm_plan_info(on)["tile_overflow"] >= 1
            G.spmm_plan_destroy(on)
            G.spmm_plan_destroy(off)

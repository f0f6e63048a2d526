"""GPU parity of graph construction and the backward pieces, through the C ABI:
edge list -> CSR (bit-exact), transposed plans (their products, bit-exact on
rows walked whole), max-pool backward (bit-exact) and the autograd wrapper."""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gnn_sparse_dense_amd as G
    from tests.gpu_helpers import DEV, check, gpu_run, log, make_plan, to_dev


def _edges(rng, E, M, K, weighted=True):
    r = rng.integers(0, M, E)
    c = rng.integers(0, K, E)
    dup = rng.random(E) < 0.05                      # some exact duplicate edges
    r[1:][dup[1:]] = r[:-1][dup[1:]]
    c[1:][dup[1:]] = c[:-1][dup[1:]]
    v = rng.random(E, dtype=np.float32) if weighted else None
    return r, c, v


@pytest.mark.parametrize("E,M,K", [(0, 10, 10), (1, 1, 1), (5000, 300, 200), (1_500_000, 200_000, 150_000)])
def test_coo_to_csr_matches_oracle(orc, E, M, K):
    rng = np.random.default_rng(E + M)
    r, c, v = _edges(rng, E, M, K)
    log(f"coo->csr E={E} M={M} K={K}")
    rp, co, vo = G.spmm_coo_to_csr(torch.from_numpy(r).to(DEV), torch.from_numpy(c).to(DEV),
                                   torch.from_numpy(v).to(DEV), M, K)
    ref = orc.coo_to_csr(r, c, v, M, K)
    assert np.array_equal(rp.cpu().numpy(), ref[0])
    assert np.array_equal(co.cpu().numpy(), ref[1])
    assert np.array_equal(vo.cpu().numpy().view(np.uint32), ref[2].view(np.uint32))
    # unweighted
    rp2, co2, vo2 = G.spmm_coo_to_csr(torch.from_numpy(r).to(DEV), torch.from_numpy(c).to(DEV), None, M, K)
    assert vo2 is None and np.array_equal(co2.cpu().numpy(), ref[1])


def test_coo_to_csr_rejects_bad_edges(orc):
    r = np.array([0, 2, 5, 1], np.int64)
    c = np.array([0, 1, 1, 9], np.int64)
    with pytest.raises(G.SpmmError) as ei:
        G.spmm_coo_to_csr(torch.from_numpy(r).to(DEV), torch.from_numpy(c).to(DEV), None, 4, 4)
    assert ei.value.status == G.SPMM_E_BAD_CSR and "edge 2" in str(ei.value)


def test_from_edge_index_product(orc):
    rng = np.random.default_rng(5)
    M, K = 4000, 3000
    r, c, v = _edges(rng, 30_000, M, K)
    ei = torch.from_numpy(np.stack([r, c])).to(DEV)
    adj = G.SparseAdj.from_edge_index(ei, M, torch.from_numpy(v).to(DEV), num_cols=K)
    rp, co, vo = orc.coo_to_csr(r, c, v, M, K)
    g = W.Graph("e", M, K, rp, co, vo)
    B = rng.standard_normal((K, 24)).astype(np.float32)
    Bd = torch.from_numpy(B).to(DEV)
    for red in ("sum", "mean", "max"):
        out = adj.reduce(Bd, red)
        torch.cuda.synchronize()
        C, arg = (out[0].cpu().numpy(), out[1].cpu().numpy()) if red == "max" else (out.cpu().numpy(), None)
        check(orc, g, B, red, C, arg, exact_rows=np.arange(M), what=f"from_edge_index {red}")
    adj.close()


CASES = [("road", 40_000), ("powerlaw", 60_000), ("community", 6_000), ("random", 0)]


@pytest.mark.parametrize("name,M", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("scale", [0, 1])
def test_transposed_plan_product(orc, name, M, scale):
    rng = np.random.default_rng(17 + scale)
    if name == "random":
        g = W.random_csr(rng, 5000, 3500, mean_deg=6.0, empty_frac=0.1, dup_frac=0.1, shuffle_rows=True)
    else:
        g = W.make_graph(name, M=M)
    log(f"transpose {name} M={g.M} nnz={g.nnz} scale={scale}")
    plan = make_plan(g)
    pt = G.spmm_plan_transpose(plan, scale)
    info = G.spmm_plan_info(pt)
    assert (info["M"], info["K"], info["nnz"]) == (g.K, g.M, g.nnz)
    assert info["has_val"] == int(g.val is not None or scale == 1)
    rt, ct, vt = orc.transpose(g.rowptr, g.col, g.val, g.M, g.K, scale=bool(scale))
    gt = W.Graph("t", g.K, g.M, rt, ct, vt if (g.val is not None or scale) else None)
    N = 32
    Gm = rng.standard_normal((g.M, N)).astype(np.float32)
    _, _, _, Gd = to_dev(gt, Gm)
    C, _ = gpu_run(pt, g.K, Gd, "sum")
    light = G.spmm_plan_partition(pt)["light"]
    check(orc, gt, Gm, "sum", C, None, exact_rows=light, what=f"transpose {name} scale={scale}")
    G.spmm_plan_destroy(pt)
    G.spmm_plan_destroy(plan)


@pytest.mark.parametrize("N", [16, 13, 64, 5, 130])
def test_max_backward_bit_exact(orc, N):
    rng = np.random.default_rng(N)
    g = W.random_csr(rng, 6000, 4500, mean_deg=7.0, empty_frac=0.1, dup_frac=0.2, shuffle_rows=True,
                     weighted=False, heavy_rows=3, heavy_deg=900)
    B = rng.integers(0, 5, size=(g.K, N)).astype(np.float32)     # many ties
    plan = make_plan(g)
    _, _, _, Bd = to_dev(g, B)
    C, arg = gpu_run(plan, g.M, Bd, "max")
    check(orc, g, B, "max", C, arg, what=f"forward max N={N}")
    dC = rng.standard_normal((g.M, N)).astype(np.float32)
    pt = G.spmm_plan_transpose(plan, 0)
    dB = torch.full((g.K, N), float("nan"), dtype=torch.float32, device=DEV)
    G.spmm_max_backward(pt, torch.from_numpy(arg).to(DEV), torch.from_numpy(dC).to(DEV), dB, N)
    torch.cuda.synchronize()
    ref = orc.max_backward(arg, dC, g.M, g.K)
    got = dB.cpu().numpy()
    log(f"max backward N={N}: {int((got != ref).sum())} differences")
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    # weighted transposes are refused
    gw = W.random_csr(rng, 100, 80, mean_deg=3.0)
    pw = make_plan(gw)
    ptw = G.spmm_plan_transpose(pw, 0)
    with pytest.raises(G.SpmmError) as ei:
        G.spmm_max_backward(ptw, torch.zeros((100, N), dtype=torch.int64, device=DEV),
                            torch.zeros((100, N), device=DEV), torch.zeros((80, N), device=DEV), N)
    assert ei.value.status == G.SPMM_E_UNSUPPORTED
    for p in (pt, plan, ptw, pw):
        G.spmm_plan_destroy(p)


@pytest.mark.parametrize("reduce", ["sum", "mean", "max"])
def test_autograd_layer(orc, reduce):
    rng = np.random.default_rng(99)
    g = W.random_csr(rng, 3000, 2500, mean_deg=5.0, empty_frac=0.1, dup_frac=0.05,
                     weighted=(reduce != "max"))
    rowptr, col, val, _ = to_dev(g)
    adj = G.SparseAdj(rowptr, col, val, num_cols=g.K)
    B = rng.standard_normal((g.K, 20)).astype(np.float32)
    Bt = torch.from_numpy(B).to(DEV).requires_grad_(True)
    out = G.aggregate(adj, Bt, reduce)
    C = out[0] if reduce == "max" else out
    dC = rng.standard_normal((g.M, 20)).astype(np.float32)
    C.backward(torch.from_numpy(dC).to(DEV))
    torch.cuda.synchronize()
    dB = Bt.grad.cpu().numpy()
    if reduce == "max":
        ref = orc.max_backward(out[1].cpu().numpy(), dC, g.M, g.K)
        assert np.array_equal(dB.view(np.uint32), ref.view(np.uint32))
    else:
        rt, ct, vt = orc.transpose(g.rowptr, g.col, g.val, g.M, g.K, scale=(reduce == "mean"))
        gt = W.Graph("t", g.K, g.M, rt, ct, vt)
        check(orc, gt, dC, "sum", dB, None, exact_rows=np.arange(g.K), what=f"autograd {reduce}")
    adj.close()


def test_backward_random_sweep(orc):
    """30 seeded random graphs (random shapes, duplicates, empty and heavy
    rows, weighted or not): edge list -> CSR bit-exact, the transposed plan
    (plain and 1/deg-scaled) through its products, and, for unweighted
    graphs, the max-pool backward bit-exact."""
    rng = np.random.default_rng(777)
    for case in range(30):
        M, K = int(rng.integers(1, 5000)), int(rng.integers(1, 5000))
        weighted = bool(rng.random() < 0.5)
        heavy = int(rng.integers(0, 4))
        g = W.random_csr(rng, M, K, mean_deg=float(rng.uniform(0.5, 20.0)), empty_frac=float(rng.uniform(0, 0.3)),
                         dup_frac=float(rng.uniform(0, 0.3)), shuffle_rows=bool(rng.random() < 0.5),
                         weighted=weighted, heavy_rows=heavy, heavy_deg=int(rng.integers(200, 2000)) if heavy else 0)
        N = int(rng.choice([1, 3, 16, 33, 64, 130]))
        what = f"backward case {case}: M={M} K={K} nnz={g.nnz} N={N} weighted={weighted}"
        log(what)
        # edge list -> CSR: the CSR's entries as an edge list, shuffled
        rows = np.repeat(np.arange(M), g.degrees())
        sh = rng.permutation(g.nnz)
        r, c = rows[sh], g.col[sh]
        v = None if g.val is None else g.val[sh]
        rp, co, vo = G.spmm_coo_to_csr(torch.from_numpy(r).to(DEV), torch.from_numpy(c).to(DEV),
                                       None if v is None else torch.from_numpy(v).to(DEV), M, K)
        ref = orc.coo_to_csr(r, c, v, M, K)
        assert np.array_equal(rp.cpu().numpy(), ref[0]) and np.array_equal(co.cpu().numpy(), ref[1]), what
        if v is not None:
            assert np.array_equal(vo.cpu().numpy().view(np.uint32), ref[2].view(np.uint32)), what
        plan = make_plan(g)
        for scale in (0, 1):
            pt = G.spmm_plan_transpose(plan, scale)
            rt, ct, vt = orc.transpose(g.rowptr, g.col, g.val, g.M, g.K, scale=bool(scale))
            gt = W.Graph("t", g.K, g.M, rt, ct, vt if (g.val is not None or scale) else None)
            Gm = rng.standard_normal((g.M, N)).astype(np.float32)
            _, _, _, Gd = to_dev(gt, Gm)
            C, _ = gpu_run(pt, g.K, Gd, "sum")
            light = G.spmm_plan_partition(pt)["light"]
            check(orc, gt, Gm, "sum", C, None, exact_rows=light, what=f"{what} transpose scale={scale}")
            if scale == 0 and not weighted:
                B = rng.integers(0, 4, size=(g.K, N)).astype(np.float32)
                _, _, _, Bd = to_dev(g, B)
                Cm, arg = gpu_run(plan, g.M, Bd, "max")
                dC = rng.standard_normal((g.M, N)).astype(np.float32)
                dB = torch.full((g.K, N), float("nan"), dtype=torch.float32, device=DEV)
                G.spmm_max_backward(pt, torch.from_numpy(arg).to(DEV), torch.from_numpy(dC).to(DEV), dB, N)
                torch.cuda.synchronize()
                refb = orc.max_backward(arg, dC, g.M, g.K)
                assert np.array_equal(dB.cpu().numpy().view(np.uint32), refb.view(np.uint32)), what
            G.spmm_plan_destroy(pt)
        G.spmm_plan_destroy(plan)


def test_max_backward_offset_pointers(orc):
    """dC, argmax and dB one element past a 16-byte boundary: float4 lanes on
    4-byte aligned rows, the same bits as the oracle, guards untouched."""
    rng = np.random.default_rng(77)
    N = 33
    g = W.random_csr(rng, 3000, 2500, mean_deg=6.0, empty_frac=0.1, weighted=False)
    B = rng.integers(0, 4, size=(g.K, N)).astype(np.float32)
    plan = make_plan(g)
    _, _, _, Bd = to_dev(g, B)
    _, arg = gpu_run(plan, g.M, Bd, "max")
    dC = rng.standard_normal((g.M, N)).astype(np.float32)
    pt = G.spmm_plan_transpose(plan, 0)
    abig = torch.empty(g.M * N + 1, dtype=torch.int64, device=DEV)
    av = abig[1:].view(g.M, N)
    av.copy_(torch.from_numpy(arg))
    cbig = torch.empty(g.M * N + 1, dtype=torch.float32, device=DEV)
    cv = cbig[1:].view(g.M, N)
    cv.copy_(torch.from_numpy(dC))
    dbig = torch.full((g.K * N + 2,), float("nan"), dtype=torch.float32, device=DEV)
    dv = dbig[1:-1].view(g.K, N)
    G.spmm_max_backward(pt, av, cv, dv, N)
    torch.cuda.synchronize()
    ref = orc.max_backward(arg, dC, g.M, g.K)
    assert np.array_equal(dv.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    assert np.isnan(dbig[0].item()) and np.isnan(dbig[-1].item())
    G.spmm_plan_destroy(pt)
    G.spmm_plan_destroy(plan)

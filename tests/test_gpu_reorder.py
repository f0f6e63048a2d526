"""GPU parity of the locality reordering (reverse Cuthill-McKee) and of the
permuted plan P A P^T, through the C ABI.  The permutation is integer work:
bit-exact against the oracle.  The permuted plan is checked through its
products, bit-exact against the fused oracle over the oracle's own P A P^T
(any difference in the permuted rows or their entry order changes bits)."""
import os

import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gnn_sparse_dense_amd as G
    from tests.gpu_helpers import DEV, check, gpu_run, log, make_plan, to_dev


def _golden():
    kv = {}
    for line in open(os.path.join(os.path.dirname(__file__), "golden", "rcm_hand.txt")):
        if line.strip() and not line.startswith("#"):
            k, *v = line.split()
            kv[k] = np.array(v, np.int64)
    return kv


def rcm_and_check(orc, g, what):
    plan = make_plan(g)
    perm = G.spmm_plan_reorder(plan)
    torch.cuda.synchronize()
    got = perm.cpu().numpy()
    ref = orc.rcm(g.rowptr, g.col, g.M)
    log(f"{what}: M={g.M} nnz={g.nnz}, {int((got != ref).sum())} positions differ")
    assert np.array_equal(got, ref), f"{what}: RCM differs"
    return plan, perm, ref


def permuted_products(orc, g, plan, perm, ref_perm, N, reduces=("sum", "mean", "max"), exact=True):
    pp = G.spmm_plan_permute(plan, perm)
    rp, cp, vp = orc.permute(g.rowptr, g.col, g.val, g.M, ref_perm)
    gp = W.Graph("p", g.M, g.M, rp, cp, vp)
    rng = np.random.default_rng(N)
    B = rng.standard_normal((g.K, N)).astype(np.float32)
    Bp = np.ascontiguousarray(B[ref_perm])
    Bpd = torch.from_numpy(Bp).to(DEV)
    info = G.spmm_plan_info(pp)
    assert (info["M"], info["K"], info["nnz"]) == (g.M, g.K, g.nnz)
    for red in reduces:
        C, arg = gpu_run(pp, g.M, Bpd, red)
        check(orc, gp, Bp, red, C, arg, exact_rows=(np.arange(g.M) if exact and not info["n_seg"] else None),
              what=f"permuted {red}")
    G.spmm_plan_destroy(pp)


def test_reorder_golden(orc):
    kv = _golden()
    M = kv["rowptr"].size - 1
    g = W.Graph("golden", M, M, kv["rowptr"], kv["col"], np.arange(1, 10, dtype=np.float32))
    plan, perm, _ = rcm_and_check(orc, g, "golden")
    assert np.array_equal(perm.cpu().numpy(), kv["perm"])
    permuted_products(orc, g, plan, perm, kv["perm"], 8)
    G.spmm_plan_destroy(plan)


def _alternating_levels(seed):
    """Breadth-first levels that alternate between a few nodes and thousands:
    short chains joined through wide layers (5,000 then 3,000 nodes, each
    wide node linked to both chain ends around it), one direction per entry,
    under random ids, so that the level kernel hands wide levels to the
    multi-block path and takes the chains back up after them."""
    rng = np.random.default_rng(seed)
    rows, cols = [], []
    nid = 0

    def new(n):
        nonlocal nid
        ids = np.arange(nid, nid + n)
        nid += n
        return ids

    def link(a, b):
        rows.append(np.asarray(a).ravel())
        cols.append(np.asarray(b).ravel())

    chain = new(3)
    link(chain[:-1], chain[1:])
    for width in (5000, 3000, 1500):
        wide = new(width)
        nxt = new(3)
        link(np.full(width, chain[-1]), wide)
        link(wide, np.full(width, nxt[0]))
        # a few links inside the wide layer
        a = rng.choice(wide, 200)
        link(a, rng.choice(wide, 200))
        link(nxt[:-1], nxt[1:])
        chain = nxt
    M = nid
    r, c = np.concatenate(rows), np.concatenate(cols)
    keep = r != c
    rowptr, col, _ = W.csr_from_pairs(M, r[keep], c[keep])
    g = W.Graph("alternating", M, M, rowptr, col, None)
    return W.relabel(g, seed)


CASES = [
    ("alternating-levels", lambda: _alternating_levels(75)),
    ("irregular", lambda: W.random_csr(np.random.default_rng(70), 3000, 3000, mean_deg=2.5, empty_frac=0.2,
                                       dup_frac=0.2, shuffle_rows=True)),
    ("road-relabelled", lambda: W.relabel(W.make_graph("road", M=60_000), 71)),
    ("community-relabelled", lambda: W.relabel(W.make_graph("community", M=8_000), 72)),
    ("powerlaw", lambda: W.make_graph("powerlaw", M=60_000)),
    ("knn-relabelled", lambda: W.relabel(W.knn_line(20_000, 10), 73)),
    ("diffusion", lambda: W.make_graph("diffusion", M=40_000)),
]


@pytest.mark.parametrize("name,make", CASES, ids=[c[0] for c in CASES])
def test_reorder_matches_oracle(orc, name, make):
    g = make()
    plan, perm, ref = rcm_and_check(orc, g, name)
    permuted_products(orc, g, plan, perm, ref, 16 if name != "community-relabelled" else 128)
    G.spmm_plan_destroy(plan)


def test_reorder_full_road_relabelled(orc):
    g = W.relabel(W.make_graph("road"), 74)
    plan, perm, ref = rcm_and_check(orc, g, "road 1M relabelled")
    rows = np.repeat(np.arange(g.M), g.degrees())
    pos = np.empty(g.M, np.int64)
    pos[ref] = np.arange(g.M)
    bw_before = np.abs(rows - g.col).max()
    bw_after = np.abs(pos[rows] - pos[g.col]).max()
    log(f"road 1M: bandwidth {bw_before} -> {bw_after}")
    assert bw_after < bw_before // 10
    G.spmm_plan_destroy(plan)


def test_reorder_errors(orc):
    rng = np.random.default_rng(75)
    g = W.random_csr(rng, 40, 30, mean_deg=3.0)
    plan = make_plan(g)
    with pytest.raises(G.SpmmError) as ei:
        G.spmm_plan_reorder(plan)
    assert ei.value.status == G.SPMM_E_INVALID_ARG
    G.spmm_plan_destroy(plan)
    sq = W.random_csr(rng, 40, 40, mean_deg=3.0)
    plan = make_plan(sq)
    with pytest.raises(G.SpmmError) as ei:
        G.spmm_plan_reorder(plan, 7)
    assert ei.value.status == G.SPMM_E_INVALID_ARG
    for bad in (np.r_[np.arange(39), 0], np.r_[np.arange(39), 40], np.r_[np.arange(39), -1]):
        with pytest.raises(G.SpmmError) as ei:
            G.spmm_plan_permute(plan, torch.from_numpy(bad.astype(np.int64)).to(DEV))
        assert ei.value.status == G.SPMM_E_INVALID_ARG
    ident = torch.arange(40, dtype=torch.int64, device=DEV)
    pp = G.spmm_plan_permute(plan, ident)
    B = rng.standard_normal((40, 8)).astype(np.float32)
    C, _ = gpu_run(pp, 40, torch.from_numpy(B).to(DEV), "sum")
    rp, cp, vp = orc.permute(sq.rowptr, sq.col, sq.val, 40, np.arange(40))
    check(orc, W.Graph("i", 40, 40, rp, cp, vp), B, "sum", C, None, exact_rows=np.arange(40), what="identity")
    G.spmm_plan_destroy(pp)
    G.spmm_plan_destroy(plan)
    empty = W.Graph("e", 5, 5, np.zeros(6, np.int64), np.zeros(0, np.int64), None)
    plan, perm, ref = rcm_and_check(orc, empty, "no entries")
    G.spmm_plan_destroy(plan)


def test_sparse_adj_reordered_roundtrip(orc):
    g = W.relabel(W.make_graph("road", M=20_000), 77)
    rowptr, col, val, _ = to_dev(g)
    adj = G.SparseAdj(rowptr, col, val, num_cols=g.K)
    radj, perm = adj.reordered()
    rng = np.random.default_rng(78)
    B = torch.from_numpy(rng.standard_normal((g.K, 32)).astype(np.float32)).to(DEV)
    C = adj.reduce(B, "sum")
    Cp = radj.reduce(B[perm].contiguous(), "sum")
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(g.M, device=DEV)
    got = Cp[inv].cpu().numpy()
    check(orc, g, B.cpu().numpy(), "sum", got, None, what="reordered round trip")
    f = radj.features(2)
    assert f["n"] == g.M and f["nnz"] == g.nnz
    assert f["mean_bandwidth"] < adj.features(2)["mean_bandwidth"] / 10
    radj.close()
    adj.close()


def _random_square(rng):
    """A random square graph of one of several structures, under random ids
    or not: irregular CSR (components, duplicates, self loops, empty rows),
    communities, a band, a kNN line, or chains joined through wide layers."""
    kind = int(rng.integers(5))
    if kind == 0:
        M = int(rng.integers(1, 6000))
        g = W.random_csr(rng, M, M, mean_deg=float(rng.uniform(0.3, 12.0)), empty_frac=float(rng.uniform(0, 0.4)),
                         dup_frac=float(rng.uniform(0, 0.3)), shuffle_rows=bool(rng.random() < 0.5))
    elif kind == 1:
        g = W.make_graph("community", M=int(rng.integers(256, 6000)))
    elif kind == 2:
        g = W.make_graph("road", M=int(rng.integers(600, 30_000)))
    elif kind == 3:
        g = W.knn_line(int(rng.integers(20, 20_000)), int(rng.integers(1, 12)))
    else:
        return _alternating_levels(int(rng.integers(1 << 30)))
    return W.relabel(g, int(rng.integers(1 << 30))) if rng.random() < 0.6 else g


def test_reorder_random_sweep(orc):
    """40 seeded random square graphs: the permutation bit-exact against the
    oracle every time (level sizes from 1 to thousands, so both the LDS level
    kernel and the multi-block path run, and hand levels to each other)."""
    rng = np.random.default_rng(4096)
    for case in range(40):
        g = _random_square(rng)
        plan, perm, ref = rcm_and_check(orc, g, f"random square graph {case}")
        G.spmm_plan_destroy(plan)

"""Pins of the CPU oracle against facts fixed outside it.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees with something the pages or the mathematics fix:

* brute-force dense float64 products (duplicates accumulated into the dense
  matrix) and scipy's CSR product, both within Higham's recursive-summation
  bound gamma_n * sum|a*b|;
* identity adjacency returns B bit for bit, argmax = own index;
* B = ones returns the (weighted) row degree; mean * deg recovers sum;
* empty rows reduce to 0 and (0, -1) (graph-spmm card, API table);
* max / argmax from numpy's max and first-occurrence argmax over the stored
  entries, with ties forced by small-integer features (graph-spmm card,
  "Correctness": max is checked against a walk over each row's stored
  entries, so duplicates count);
* val = NULL equals an explicit all-ones weight array bit for bit (card,
  "Correctness");
* the row split against a hand-enumerated case and its tiling invariants;
* degree descriptors against closed forms and numpy's population std;
* the MAC-job gap against ParamSpMM Table 2.

tests/test_oracle.py runs every pin on the real oracle; tests/test_oracle_mutants.py
runs them on oracle builds with a planted mistake and requires some pin to fail.
"""
from __future__ import annotations

import math
import os

import numpy as np

import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
U = 2.0 ** -24          # fp32 unit roundoff


def gamma(n):
    n = np.asarray(n, dtype=np.float64)
    return n * U / (1.0 - n * U)


def _dense(g: W.Graph) -> np.ndarray:
    A = np.zeros((g.M, g.K), dtype=np.float64)
    rows = np.repeat(np.arange(g.M), g.degrees())
    vals = np.ones(g.nnz) if g.val is None else g.val.astype(np.float64)
    np.add.at(A, (rows, g.col), vals)            # duplicates accumulate
    return A


def _small_graphs():
    rng = np.random.default_rng(20240601)
    out = []
    for it in range(8):
        M = int(rng.integers(1, 65))
        K = int(rng.integers(1, 65))
        out.append(W.random_csr(rng, M, K, mean_deg=float(rng.uniform(0.5, 12)),
                                empty_frac=0.15, dup_frac=0.2 if it % 2 else 0.0,
                                shuffle_rows=bool(it % 3 == 0), weighted=bool(it % 4 != 1)))
    return out


def _bound_check(C, ref, S, deg, what, mean=False):
    n = np.maximum(deg, 1)[:, None]
    if mean:
        tol = (gamma(n + 2) * S) / n
    else:
        tol = gamma(n + 1) * S
    err = np.abs(C.astype(np.float64) - ref)
    bad = err > tol + 1e-300
    assert not bad.any(), f"{what}: {int(bad.sum())} entries outside the recursive-summation bound"


def pin_dense_bruteforce(orc):
    rng = np.random.default_rng(7)
    for g in _small_graphs():
        N = int(rng.integers(1, 9))
        B = rng.standard_normal((g.K, N)).astype(np.float32)
        ref = _dense(g) @ B.astype(np.float64)
        Sabs = np.abs(_dense_abs(g)) @ np.abs(B.astype(np.float64))
        deg = g.degrees()
        for fused in (False, True):
            C = orc.spmm(g.rowptr, g.col, g.val, g.M, g.K, B, "sum", fused=fused)
            _bound_check(C, ref, Sabs, deg, f"sum fused={fused}")
            Cm = orc.spmm(g.rowptr, g.col, g.val, g.M, g.K, B, "mean", fused=fused)
            refm = np.where(deg[:, None] > 0, ref / np.maximum(deg, 1)[:, None], 0.0)
            _bound_check(Cm, refm, Sabs, deg, f"mean fused={fused}", mean=True)


def _dense_abs(g: W.Graph) -> np.ndarray:
    A = np.zeros((g.M, g.K), dtype=np.float64)
    rows = np.repeat(np.arange(g.M), g.degrees())
    vals = np.ones(g.nnz) if g.val is None else np.abs(g.val.astype(np.float64))
    np.add.at(A, (rows, g.col), vals)
    return A


def pin_scipy_product(orc):
    import scipy.sparse as sp
    rng = np.random.default_rng(11)
    g = W.random_csr(rng, 300, 250, mean_deg=9.0, empty_frac=0.05, dup_frac=0.1)
    for N in (1, 5, 33):
        B = rng.standard_normal((g.K, N)).astype(np.float32)
        A = sp.csr_matrix((g.val.astype(np.float64), g.col, g.rowptr), shape=(g.M, g.K))
        ref = np.asarray(A @ B.astype(np.float64))
        Aabs = sp.csr_matrix((np.abs(g.val.astype(np.float64)), g.col, g.rowptr), shape=(g.M, g.K))
        S = np.asarray(Aabs @ np.abs(B.astype(np.float64)))
        C = orc.spmm(g.rowptr, g.col, g.val, g.M, g.K, B, "sum")
        _bound_check(C, ref, S, g.degrees(), f"scipy N={N}")
        S2 = orc.sumabs(g.rowptr, g.col, g.val, g.M, B)
        assert np.allclose(S2, S, rtol=1e-12, atol=0), "sumabs differs from |A| @ |B|"


def pin_identity(orc):
    rng = np.random.default_rng(3)
    M = 37
    B = rng.standard_normal((M, 7)).astype(np.float32)
    rowptr = np.arange(M + 1, dtype=np.int64)
    col = np.arange(M, dtype=np.int64)
    for val in (None, np.ones(M, np.float32)):
        for red in ("sum", "mean"):
            C = orc.spmm(rowptr, col, val, M, M, B, red)
            assert np.array_equal(C.view(np.uint32), B.view(np.uint32)), f"identity {red}"
        C, arg = orc.spmm(rowptr, col, val, M, M, B, "max")
        assert np.array_equal(C.view(np.uint32), B.view(np.uint32)), "identity max"
        assert np.array_equal(arg, np.repeat(np.arange(M)[:, None], 7, axis=1)), "identity argmax"


def pin_ones(orc):
    rng = np.random.default_rng(5)
    g = W.random_csr(rng, 120, 90, mean_deg=6.0, empty_frac=0.1, dup_frac=0.1, weighted=False)
    B = np.ones((g.K, 4), np.float32)
    deg = g.degrees().astype(np.float32)
    C = orc.spmm(g.rowptr, g.col, None, g.M, g.K, B, "sum")
    assert np.array_equal(C, np.repeat(deg[:, None], 4, axis=1)), "unweighted ones -> degree"
    gw = W.random_csr(rng, 120, 90, mean_deg=6.0, empty_frac=0.1, dup_frac=0.1, weighted=True)
    Cw = orc.spmm(gw.rowptr, gw.col, gw.val, gw.M, gw.K, B, "sum")
    for i in range(gw.M):
        a, b = gw.rowptr[i], gw.rowptr[i + 1]
        exact = math.fsum(float(v) for v in gw.val[a:b])
        tol = float(gamma(b - a + 1)) * math.fsum(abs(float(v)) for v in gw.val[a:b])
        assert np.all(np.abs(Cw[i].astype(np.float64) - exact) <= tol), f"weighted degree row {i}"
    Cm = orc.spmm(g.rowptr, g.col, None, g.M, g.K, B, "mean")
    nz = deg > 0
    assert np.all(Cm[nz] == 1.0) and np.all(Cm[~nz] == 0.0), "unweighted ones mean -> 1"


def pin_empty_rows(orc):
    rowptr = np.array([0, 0, 2, 2, 3, 3], np.int64)
    col = np.array([1, 0, 2], np.int64)
    val = np.array([0.5, -2.0, 3.0], np.float32)
    B = np.array([[1.0, -1.0], [2.0, 4.0], [-3.0, 0.25]], np.float32)
    M, K = 5, 3
    empty = np.array([True, False, True, False, True])
    for red in ("sum", "mean"):
        C = orc.spmm(rowptr, col, val, M, K, B, red)
        assert np.all(C[empty].view(np.uint32) == 0), f"{red}: empty rows must be +0"
    C, arg = orc.spmm(rowptr, col, val, M, K, B, "max")
    assert np.all(C[empty].view(np.uint32) == 0) and np.all(arg[empty] == -1), "max empty -> (0,-1)"
    # row 1: entries (col 1, 0.5) and (col 0, -2.0); row 3: (col 2, 3.0)
    assert np.array_equal(C[1], np.float32([max(0.5 * 2.0, -2.0 * 1.0), max(0.5 * 4.0, -2.0 * -1.0)]))
    assert np.array_equal(arg[1], [1, 1]), "first maximum wins (0.5*4 == -2*-1)"
    assert np.array_equal(C[3], np.float32([-9.0, 0.75])) and np.array_equal(arg[3], [2, 2])
    Cs = orc.spmm(rowptr, col, val, M, K, B, "sum")
    assert np.array_equal(Cs[1], np.float32([1.0 - 2.0, 2.0 + 2.0]))
    Cm = orc.spmm(rowptr, col, val, M, K, B, "mean")
    assert np.array_equal(Cm[1], np.float32([-0.5, 2.0]))


def pin_max_numpy(orc):
    rng = np.random.default_rng(13)
    for it in range(6):
        g = W.random_csr(rng, 80, 60, mean_deg=7.0, empty_frac=0.1, dup_frac=0.25,
                         shuffle_rows=bool(it % 2), weighted=bool(it % 3))
        if g.val is not None and it % 2:
            g.val = rng.choice(np.float32([0.0, 0.5, 1.0, -1.0]), size=g.nnz).astype(np.float32)
        N = 6
        B = rng.integers(0, 3, size=(g.K, N)).astype(np.float32)       # ties everywhere
        if it >= 3:
            B = rng.standard_normal((g.K, N)).astype(np.float32)
        C, arg = orc.spmm(g.rowptr, g.col, g.val, g.M, g.K, B, "max")
        for i in range(g.M):
            a, b = g.rowptr[i], g.rowptr[i + 1]
            if a == b:
                continue
            cols = g.col[a:b]
            t = B[cols]                                                  # [deg, N] fp32
            if g.val is not None:
                t = (g.val[a:b, None] * t).astype(np.float32)
            j = np.argmax(t, axis=0)                                     # first occurrence
            first_max = t[j, np.arange(N)]                               # its exact bits (+0 vs -0)
            assert np.array_equal(C[i].view(np.uint32), first_max.view(np.uint32)), f"max row {i}"
            assert np.array_equal(arg[i], cols[j]), f"argmax row {i}"


def pin_val_null_is_ones(orc):
    rng = np.random.default_rng(17)
    g = W.random_csr(rng, 200, 150, mean_deg=9.0, dup_frac=0.1, weighted=False)
    B = rng.standard_normal((g.K, 12)).astype(np.float32)
    ones = np.ones(g.nnz, np.float32)
    for red in ("sum", "mean"):
        for fused in (False, True):
            a = orc.spmm(g.rowptr, g.col, None, g.M, g.K, B, red, fused=fused)
            b = orc.spmm(g.rowptr, g.col, ones, g.M, g.K, B, red, fused=fused)
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"val=NULL {red}"
    a, ia = orc.spmm(g.rowptr, g.col, None, g.M, g.K, B, "max")
    b, ib = orc.spmm(g.rowptr, g.col, ones, g.M, g.K, B, "max")
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32)) and np.array_equal(ia, ib)


def pin_mean_sum_relation(orc):
    rng = np.random.default_rng(19)
    g = W.random_csr(rng, 150, 100, mean_deg=5.0, empty_frac=0.2)
    B = rng.standard_normal((g.K, 9)).astype(np.float32)
    S = orc.spmm(g.rowptr, g.col, g.val, g.M, g.K, B, "sum")
    Mn = orc.spmm(g.rowptr, g.col, g.val, g.M, g.K, B, "mean")
    deg = g.degrees()
    for i in range(g.M):
        if deg[i] == 0:
            assert np.all(Mn[i] == 0)
        else:
            assert np.array_equal(Mn[i], (S[i] / np.float32(deg[i])).astype(np.float32)), f"mean row {i}"


def pin_row_subset(orc):
    rng = np.random.default_rng(23)
    g = W.random_csr(rng, 90, 70, mean_deg=6.0, dup_frac=0.1)
    B = rng.standard_normal((g.K, 5)).astype(np.float32)
    rows = np.array([89, 0, 17, 17, 42], np.int64)
    for red in ("sum", "mean"):
        full = orc.spmm(g.rowptr, g.col, g.val, g.M, g.K, B, red)
        sub = orc.spmm(g.rowptr, g.col, g.val, g.M, g.K, B, red, rows=rows)
        assert np.array_equal(full[rows], sub), f"row subset {red}"
    full, fa = orc.spmm(g.rowptr, g.col, g.val, g.M, g.K, B, "max")
    sub, sa = orc.spmm(g.rowptr, g.col, g.val, g.M, g.K, B, "max", rows=rows)
    assert np.array_equal(full[rows], sub) and np.array_equal(fa[rows], sa)


def _read_partition_golden():
    segs, light = [], []
    with open(os.path.join(GOLDEN, "partition_hand.txt")) as f:
        for line in f:
            line = line.split("#")[0].split()
            if not line:
                continue
            if line[0] == "seg":
                segs.append(tuple(int(x) for x in line[1:4]))
            elif line[0] == "light":
                light.append(int(line[1]))
    return segs, light


def pin_partition(orc):
    rowptr = np.array([0, 0, 5, 1205, 1718], np.int64)
    segs, light = _read_partition_golden()
    p = orc.partition(rowptr, 4, 512, 512)
    got = list(zip(p["seg_row"].tolist(), p["seg_begin"].tolist(), p["seg_end"].tolist()))
    assert got == segs, f"hand partition: {got}"
    assert p["light"].tolist() == light and p["n_heavy"] == 2
    # T = 0: every non-empty row is heavy; L = 1: one piece per entry
    q = orc.partition(rowptr, 4, 0, 1)
    assert q["n_heavy"] == 3 and len(q["seg_row"]) == 1718 and q["light"].tolist() == [0]
    assert np.array_equal(q["seg_begin"], np.arange(1718)) and np.array_equal(q["seg_end"], np.arange(1, 1719))
    # tiling invariants on a skewed random graph
    rng = np.random.default_rng(29)
    g = W.random_csr(rng, 500, 500, mean_deg=4.0, heavy_rows=7, heavy_deg=777)
    deg = g.degrees()
    for T, L in ((16, 16), (100, 64), (776, 777), (777, 1)):
        r = orc.partition(g.rowptr, g.M, T, L)
        heavy = np.nonzero(deg > T)[0]
        assert np.array_equal(r["light"], np.nonzero(deg <= T)[0])
        assert r["n_heavy"] == heavy.size
        sr, sb, se = r["seg_row"], r["seg_begin"], r["seg_end"]
        assert np.all(np.diff(sr) >= 0) and np.all(se > sb) and np.all(se - sb <= L)
        for h in heavy:
            m = sr == h
            assert sb[m][0] == g.rowptr[h] and se[m][-1] == g.rowptr[h + 1]
            assert np.array_equal(sb[m][1:], se[m][:-1])
            assert np.all((se[m] - sb[m])[:-1] == L)
        assert set(sr.tolist()) == set(heavy.tolist())


def pin_descriptors(orc):
    def rp(deg):
        return np.concatenate([[0], np.cumsum(deg)]).astype(np.int64)
    d = orc.descriptors(rp([10] * 50), 50)
    assert d["mean"] == 10.0 and d["cv"] == 0.0 and d["dmax"] == 10 and d["n_empty"] == 0
    d = orc.descriptors(rp([0, 2]), 2)
    assert d["mean"] == 1.0 and abs(d["cv"] - 1.0) < 1e-15 and d["n_empty"] == 1 and d["nnz"] == 2
    d = orc.descriptors(rp([1, 2, 3, 4]), 4)
    assert abs(d["cv"] - math.sqrt(1.25) / 2.5) < 1e-15 and d["dmax"] == 4
    d = orc.descriptors(rp([]), 0)
    assert d["mean"] == 0.0 and d["cv"] == 0.0 and d["nnz"] == 0
    rng = np.random.default_rng(31)
    deg = rng.zipf(2.1, size=5000).clip(0, 100000)
    d = orc.descriptors(rp(deg), deg.size)
    assert abs(d["cv"] - deg.std() / deg.mean()) <= 1e-12 * d["cv"]
    assert d["dmax"] == deg.max() and d["n_empty"] == int((deg == 0).sum())


def pin_validate(orc):
    assert orc.validate(np.array([0, 2, 3], np.int64), np.array([0, 1, 1], np.int64), 2, 2) == -1
    assert orc.validate(np.array([1, 2, 3], np.int64), np.array([0, 1, 1], np.int64), 2, 2) == 0
    assert orc.validate(np.array([0, 2, 1], np.int64), np.array([0, 1, 1], np.int64), 2, 2) == 1
    assert orc.validate(np.array([0, 2, 3], np.int64), np.array([0, 1, 2], np.int64), 2, 2) == 1
    assert orc.validate(np.array([0, 2, 3], np.int64), np.array([0, -1, 1], np.int64), 2, 2) == 0
    assert orc.validate(np.array([0, 0, 0], np.int64), np.zeros(0, np.int64), 2, 0) == -1


def pin_mac_gap(orc):
    with open(os.path.join(GOLDEN, "paramspmm_table2_mac_gap.txt")) as f:
        rows = [line.split() for line in f if line.strip() and not line.startswith("#")]
    assert len(rows) == 14
    for dim, F, omega, gap in rows:
        got = orc.mac_gap(int(dim), int(F), int(omega))
        assert got == int(gap), f"gap(dim={dim}, F={F}) = {got}, Table 2 prints {gap}"


def pin_tiny_config(orc):
    """The full tiny regime against dense float64 products."""
    w = W.make("tiny")
    g = w.graph
    B = w.B
    ref = _dense(g) @ B.astype(np.float64)
    S = _dense_abs(g) @ np.abs(B.astype(np.float64))
    C = orc.spmm(g.rowptr, g.col, g.val, g.M, g.K, B, "sum")
    _bound_check(C, ref, S, g.degrees(), "tiny sum")
    S2 = orc.sumabs(g.rowptr, g.col, g.val, g.M, B)
    assert np.allclose(S2, S, rtol=1e-12, atol=0)


def pin_coo_to_csr(orc):
    rowptr, col, val = orc.coo_to_csr([2, 0, 2, 1], [1, 3, 0, 0], np.float32([1, 2, 3, 4]), 3, 4)
    assert rowptr.tolist() == [0, 1, 2, 4] and col.tolist() == [3, 0, 1, 0] and val.tolist() == [2, 4, 1, 3]
    try:
        orc.coo_to_csr([0, 3], [0, 0], None, 3, 4)
        raise AssertionError("row 3 of 3 accepted")
    except ValueError as e:
        assert "bad edge 1" in str(e)
    import scipy.sparse as sp
    rng = np.random.default_rng(41)
    M, K, E = 300, 200, 2500
    r = rng.integers(0, M, E)
    c = rng.integers(0, K, E)
    v = rng.random(E, dtype=np.float32)
    rowptr, col, val = orc.coo_to_csr(r, c, v, M, K)
    order = np.argsort(r, kind="stable")                  # numpy's stable sort
    assert np.array_equal(rowptr, np.concatenate([[0], np.cumsum(np.bincount(r, minlength=M))]))
    assert np.array_equal(col, c[order]) and np.array_equal(val, v[order])
    B = rng.standard_normal((K, 6)).astype(np.float32)
    ref = np.asarray(sp.coo_matrix((v.astype(np.float64), (r, c)), shape=(M, K)).tocsr() @ B.astype(np.float64))
    S = np.asarray(sp.coo_matrix((np.abs(v.astype(np.float64)), (r, c)), shape=(M, K)).tocsr()
                   @ np.abs(B.astype(np.float64)))
    C = orc.spmm(rowptr, col, val, M, K, B, "sum")
    _bound_check(C, ref, S, np.diff(rowptr), "coo product")


def pin_transpose(orc):
    rng = np.random.default_rng(43)
    for weighted in (True, False):
        g = W.random_csr(rng, 150, 120, mean_deg=5.0, empty_frac=0.1, dup_frac=0.2, shuffle_rows=True,
                         weighted=weighted)
        rt, ct, vt = orc.transpose(g.rowptr, g.col, g.val, g.M, g.K)
        gt = W.Graph("t", g.K, g.M, rt, ct, vt)
        assert np.array_equal(_dense(gt), _dense(g).T), "dense transpose"
        for j in range(g.K):                                  # rows i ascend within each row
            assert np.all(np.diff(ct[rt[j]:rt[j + 1]]) >= 0)
        rtt, ctt, vtt = orc.transpose(rt, ct, vt, g.K, g.M)
        for i in range(g.M):                                  # twice = rows sorted by column, stably
            a, b = g.rowptr[i], g.rowptr[i + 1]
            o = np.argsort(g.col[a:b], kind="stable")
            assert np.array_equal(ctt[a:b], g.col[a:b][o])
            vals = np.ones(b - a, np.float32) if g.val is None else g.val[a:b]
            assert np.array_equal(vtt[a:b], vals[o])
        _, _, vs = orc.transpose(g.rowptr, g.col, g.val, g.M, g.K, scale=True)
        deg = np.diff(g.rowptr)
        a = np.ones(g.nnz, np.float32) if g.val is None else g.val
        expect = (a / np.repeat(deg, deg).astype(np.float32)).astype(np.float32)
        perm = np.argsort(g.col, kind="stable")               # entry order of the transpose
        assert np.array_equal(vs, expect[perm]), "mean-backward weights"
        # adjoint: <A B, G> == <B, A^T G>
        B = rng.standard_normal((g.K, 5)).astype(np.float32)
        Gm = rng.standard_normal((g.M, 5)).astype(np.float32)
        lhs = float(np.sum(orc.spmm(g.rowptr, g.col, g.val, g.M, g.K, B, "sum").astype(np.float64) * Gm))
        rhs = float(np.sum(B.astype(np.float64) * orc.spmm(rt, ct, vt, g.K, g.M, Gm, "sum")))
        assert abs(lhs - rhs) <= 1e-4 * (1 + abs(lhs)), (lhs, rhs)


def pin_max_backward(orc):
    argmax = np.array([[2, -1], [0, 2], [2, 2]], np.int64)
    dC = np.float32([[1.5, 7.0], [0.25, -1.0], [2.0, 0.5]])
    dB = orc.max_backward(argmax, dC, 3, 4)
    assert np.array_equal(dB, np.float32([[0.25, 0], [0, 0], [1.5 + 2.0, -1.0 + 0.5], [0, 0]]))
    rng = np.random.default_rng(47)
    g = W.random_csr(rng, 400, 250, mean_deg=6.0, empty_frac=0.1, dup_frac=0.1, weighted=False)
    B = rng.integers(0, 4, size=(g.K, 7)).astype(np.float32)
    C, arg = orc.spmm(g.rowptr, g.col, None, g.M, g.K, B, "max")
    dC = rng.standard_normal((g.M, 7)).astype(np.float32)
    dB = orc.max_backward(arg, dC, g.M, g.K)
    ref = np.zeros((g.K, 7), np.float32)
    ii, kk = np.nonzero(arg >= 0)                             # i-major order
    np.add.at(ref, (arg[ii, kk], kk), dC[ii, kk])
    assert np.array_equal(dB.view(np.uint32), ref.view(np.uint32)), "max backward vs np.add.at"
    lhs = float(np.sum(dC.astype(np.float64) * np.where(arg >= 0, C, 0)))
    rhs = float(np.sum(dB.astype(np.float64) * B))
    assert abs(lhs - rhs) <= 1e-4 * (1 + abs(lhs))


def _read_features_golden():
    kv = {}
    for line in open(os.path.join(GOLDEN, "features_hand.txt")):
        if line.startswith("#") or not line.strip():
            continue
        k, *v = line.split()
        kv[k] = v
    return kv


def pin_features(orc):
    kv = _read_features_golden()
    rp = np.array(kv["rowptr"], np.int64)
    col = np.array(kv["col"], np.int64)
    M, K = int(kv["M"][0]), int(kv["K"][0])
    for V in (1, 2, 3):
        f = orc.features(rp, col, M, K, V)
        for key in ("n_nonempty", "nnz", "dmax", "max_bandwidth", "nnz_distinct"):
            assert f[key] == int(kv[key][0]), (key, f[key])
        for key in ("delta", "mean_deg", "mean_deg_nonempty", "cv_deg", "cv_deg_nonempty", "density",
                    "mean_bandwidth"):
            assert abs(f[key] - float(kv[key][0])) <= 1e-12, (key, f[key])
        assert f["nnz_vectors"] == int(kv[f"vectors_V{V}"][0]), (V, f["nnz_vectors"])
        assert abs(f["padding_ratio"] - float(kv[f"padding_V{V}"][0])) <= 1e-12, (V, f["padding_ratio"])
    # numpy brute force on irregular graphs (duplicates, unsorted rows, empty rows)
    rng = np.random.default_rng(53)
    for V in (1, 2, 4):
        g = W.random_csr(rng, 333, 97, mean_deg=6.0, empty_frac=0.2, dup_frac=0.3, shuffle_rows=True)
        f = orc.features(g.rowptr, g.col, g.M, g.K, V)
        deg = g.degrees()
        rows = np.repeat(np.arange(g.M), deg)
        ne = deg > 0
        pairs = np.unique(rows * g.K + g.col).size
        vecs = np.unique((rows // V) * g.K + g.col).size
        assert f["nnz_distinct"] == pairs and f["nnz_vectors"] == vecs
        assert abs(f["padding_ratio"] - (1 - pairs / (vecs * V))) <= 1e-12
        assert abs(f["cv_deg_nonempty"] - np.std(deg[ne]) / np.mean(deg[ne])) <= 1e-12
        assert abs(f["cv_deg"] - np.std(deg) / np.mean(deg)) <= 1e-12
        starts = g.rowptr[:-1][ne]
        bw = np.maximum.reduceat(g.col, starts) - np.minimum.reduceat(g.col, starts)
        assert f["max_bandwidth"] == bw.max() and abs(f["mean_bandwidth"] - bw.mean()) <= 1e-9
        assert 0.0 <= f["padding_ratio"] <= 1.0 - 1.0 / V + 1e-15
    # closed cases: identical row pairs share every column (no padding), disjoint
    # row pairs share none (the largest padding of V = 2)
    same = np.array([0, 3, 6, 8, 10], np.int64)
    assert orc.features(same, np.array([1, 4, 6, 1, 4, 6, 2, 9, 2, 9]), 4, 10, 2)["padding_ratio"] == 0.0
    assert orc.features(same, np.array([1, 4, 6, 0, 5, 7, 2, 9, 3, 8]), 4, 10, 2)["padding_ratio"] == 0.5


def _read_rcm_golden():
    kv = {}
    for line in open(os.path.join(GOLDEN, "rcm_hand.txt")):
        if line.strip() and not line.startswith("#"):
            k, *v = line.split()
            kv[k] = np.array(v, np.int64)
    return kv


def _check_cuthill_mckee(rowptr, col, M, perm):
    """Verifies the defining properties of the (unreversed) Cuthill-McKee order
    q = perm[::-1] on the symmetric pattern, independently of how it was built."""
    assert np.array_equal(np.sort(perm), np.arange(M)), "not a permutation"
    rows = np.repeat(np.arange(M), np.diff(rowptr))
    off = rows != col
    a, b = rows[off], col[off]
    und = np.unique(np.concatenate([a * M + b, b * M + a])) if off.any() else np.zeros(0, np.int64)
    nbr = [[] for _ in range(M)]
    for k in und.tolist():
        nbr[k // M].append(k % M)
    deg = np.array([len(x) for x in nbr])
    q = perm[::-1]
    pos = np.empty(M, np.int64)
    pos[q] = np.arange(M)
    key = deg * (M + 1) + np.arange(M)                 # (degree, id) rank
    parent = np.full(M, -1)
    for t, v in enumerate(q.tolist()):
        earlier = [pos[u] for u in nbr[v] if pos[u] < t]
        if earlier:
            parent[v] = min(earlier)
        else:                                          # a component start: the smallest
            rest = q[t:]                               # unplaced node in (degree, id) order
            assert key[v] == key[rest].min(), f"start {v} is not the smallest remaining"
    par = parent[q]
    for t in range(1, M):
        if par[t] >= 0 and par[t - 1] >= 0:
            assert par[t] >= par[t - 1], "parents out of order"
            if par[t] == par[t - 1]:
                assert key[q[t]] > key[q[t - 1]], "siblings not in (degree, id) order"


def pin_rcm(orc):
    kv = _read_rcm_golden()
    M = kv["rowptr"].size - 1
    perm = orc.rcm(kv["rowptr"], kv["col"], M)
    assert np.array_equal(perm, kv["perm"]), f"hand RCM: {perm}"
    rp, cp, vp = orc.permute(kv["rowptr"], kv["col"], np.arange(1, 10, dtype=np.float32), M, kv["perm"])
    assert np.array_equal(rp, kv["rowptr_p"]) and np.array_equal(cp, kv["col_p"])
    assert np.array_equal(vp, kv["val_p"].astype(np.float32))
    # a shuffled path: Cuthill-McKee from an end recovers bandwidth 1
    rng = np.random.default_rng(61)
    n = 300
    lab = rng.permutation(n)
    g = W.csr_from_pairs(n, lab[:-1], lab[1:])
    p = orc.rcm(g[0], g[1], n)
    rq, cq, _ = orc.permute(g[0], g[1], None, n, p)
    assert np.abs(np.repeat(np.arange(n), np.diff(rq)) - cq).max() == 1
    # defining properties on irregular graphs (several components, duplicates, self loops)
    for seed in (62, 63):
        r = np.random.default_rng(seed)
        gr = W.random_csr(r, 400, 400, mean_deg=2.0, empty_frac=0.2, dup_frac=0.2, shuffle_rows=True)
        pr = orc.rcm(gr.rowptr, gr.col, gr.M)
        _check_cuthill_mckee(gr.rowptr, gr.col, gr.M, pr)
        # P A P^T against dense indexing; rows ascending by new column
        rq, cq, vq = orc.permute(gr.rowptr, gr.col, gr.val, gr.M, pr)
        gq = W.Graph("p", gr.M, gr.M, rq, cq, vq)
        assert np.array_equal(_dense(gq), _dense(gr)[np.ix_(pr, pr)])
        for i in range(gr.M):
            assert np.all(np.diff(cq[rq[i]:rq[i + 1]]) >= 0)


def _read_fused_golden():
    B, entries, expect = {}, [], []
    with open(os.path.join(GOLDEN, "fused_rounding_hand.txt")) as f:
        for line in f:
            t = line.split("#")[0].split()
            if not t:
                continue
            if t[0] == "B":
                B[int(t[1])] = float.fromhex(t[2])
            elif t[0] == "entry":
                entries.append((int(t[1]), int(t[2]), float.fromhex(t[3])))
            elif t[0] == "expect":
                expect.append((t[1], t[2] == "fused", int(t[3]), float.fromhex(t[4])))
    return B, entries, expect


def pin_fused_rounding(orc):
    """Plain and fused sums on a row where one rounding of the multiply-add
    and two roundings give different bits (hand-worked golden), in both entry
    orders (stored order rules)."""
    Bd, entries, expect = _read_fused_golden()
    K = len(Bd)
    M = max(r for r, _, _ in entries) + 1
    B = np.array([[Bd[k]] for k in range(K)], np.float32)
    rowptr = np.zeros(M + 1, np.int64)
    for r, _, _ in entries:
        rowptr[r + 1] += 1
    rowptr = np.cumsum(rowptr)
    col = np.array([c for _, c, _ in entries], np.int64)
    val = np.array([a for _, _, a in entries], np.float32)
    for red, fused, row, want in expect:
        C = orc.spmm(rowptr, col, val, M, K, B, red, fused=fused)
        got = np.float32(C[row, 0])
        assert got.view(np.uint32) == np.float32(want).view(np.uint32), \
            f"{red} fused={fused} row {row}: {float(got).hex()} != {want.hex()}"


ALL_PINS = [
    pin_dense_bruteforce, pin_scipy_product, pin_identity, pin_ones, pin_empty_rows,
    pin_max_numpy, pin_val_null_is_ones, pin_mean_sum_relation, pin_row_subset,
    pin_partition, pin_descriptors, pin_validate, pin_mac_gap, pin_tiny_config,
    pin_coo_to_csr, pin_transpose, pin_max_backward, pin_features, pin_rcm,
    pin_fused_rounding,
]

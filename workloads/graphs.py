"""Five synthetic graph regimes plus small random CSR matrices for edge cases.

The regimes stand in for the graph suites the source pages measure on (SNAP,
DIMACS10, OGB and the RA-SpMM / DualGCN suites), none of which are available
here.  Each follows the structural class the pages name:

* ``tiny``       -- small Poisson random graph, correctness reference.
* ``road``       -- sparse-uniform, banded locality (RA-SpMM "sparse uniform"
                    regime: mean degree < 20, CV < 1, more than 100k rows;
                    ParamSpMM's Poisson road networks).
* ``powerlaw``   -- heavy-tailed social graph with GCN normalised weights
                    (RA-SpMM "extreme-skew sparse tail"; ParamSpMM power-law).
* ``diffusion``  -- near-regular kNN-like graph, 1M nodes / 10M edges /
                    16 channels (graph-spmm card, hero caption and table).
* ``community``  -- contiguous 256-node communities with sparse inter-community
                    edges (RA-SpMM "community / locality" regime).

All randomness comes from numpy's PCG64 generator seeded per regime, with
independent child streams for structure, edge values and features, so changing
the feature width never changes the graph.  Columns are distinct and sorted
within each row for every regime.
"""
from __future__ import annotations

import dataclasses
from typing import Callable, Optional, Tuple

import numpy as np


@dataclasses.dataclass
class Graph:
    name: str
    M: int
    K: int
    rowptr: np.ndarray            # int64 [M+1]
    col: np.ndarray               # int64 [nnz]
    val: Optional[np.ndarray]     # float32 [nnz] or None (unweighted)

    @property
    def nnz(self) -> int:
        return int(self.rowptr[-1])

    def degrees(self) -> np.ndarray:
        return np.diff(self.rowptr)


@dataclasses.dataclass
class Workload:
    graph: Graph
    N: int
    B: np.ndarray                 # float32 [K, N], row-major
    reduces: Tuple[str, ...]


# name -> (M=K, N, seed, reductions).  Sizes are the full single-GPU shapes.
CONFIGS = {
    "tiny":      dict(M=2_000,     N=16,  seed=1, reduces=("sum", "mean", "max")),
    "road":      dict(M=1_000_000, N=64,  seed=2, reduces=("sum", "mean")),
    "powerlaw":  dict(M=2_000_000, N=128, seed=3, reduces=("sum",)),
    "diffusion": dict(M=1_000_000, N=16,  seed=4, reduces=("mean", "max")),
    "community": dict(M=500_000,   N=512, seed=5, reduces=("sum",)),
    # router evaluation only: a third road-like band, a third community
    # blocks, a third power-law rows over all columns
    "mixed":     dict(M=1_000_000, N=128, seed=6, reduces=("sum",)),
    # router evaluation only: k-nearest-neighbour graph of points on a line
    # (k = 10, unweighted), where two adjacent rows share most columns
    "knn":       dict(M=1_000_000, N=64,  seed=7, reduces=("sum",)),
}


def _streams(seed: int):
    ss = np.random.SeedSequence(seed)
    s_struct, s_val, s_feat = ss.spawn(3)
    return (np.random.Generator(np.random.PCG64(s_struct)),
            np.random.Generator(np.random.PCG64(s_val)),
            np.random.Generator(np.random.PCG64(s_feat)))


def _rowptr_from_deg(deg: np.ndarray) -> np.ndarray:
    rp = np.zeros(len(deg) + 1, dtype=np.int64)
    np.cumsum(deg, out=rp[1:])
    return rp


def _concat_ranges(starts: np.ndarray, lens: np.ndarray) -> np.ndarray:
    """Concatenation of arange(s, s+l) for each (s, l), vectorised."""
    lens = lens.astype(np.int64)
    total = int(lens.sum())
    if total == 0:
        return np.zeros(0, dtype=np.int64)
    first = np.cumsum(lens) - lens
    return np.repeat(starts.astype(np.int64) - first, lens) + np.arange(total, dtype=np.int64)


def _distinct_columns(rng, deg: np.ndarray, K: int,
                      draw: Callable[[np.random.Generator, np.ndarray], np.ndarray],
                      forbid_self: bool = False, max_iter: int = 1000):
    """Draw deg[i] distinct columns for every row i, sorted within the row.

    ``draw(rng, rows)`` returns one candidate column per entry of ``rows``.
    Repeated columns (and self loops when ``forbid_self``) are redrawn until
    every row is clean; only the affected rows are re-sorted each round.
    """
    deg = deg.astype(np.int64)
    rowptr = _rowptr_from_deg(deg)
    nnz = int(rowptr[-1])
    rows = np.repeat(np.arange(len(deg), dtype=np.int64), deg)
    cols = draw(rng, rows).astype(np.int64)
    sel = np.arange(nnz, dtype=np.int64)
    for _ in range(max_iter):
        if sel.size == 0:
            break
        r = rows[sel]
        c = cols[sel]
        order = np.argsort(r * np.int64(K) + c, kind="stable")
        c = c[order]                      # rows stay grouped: r[order] == r
        bad = np.zeros(sel.size, dtype=bool)
        bad[1:] = (c[1:] == c[:-1]) & (r[1:] == r[:-1])
        if forbid_self:
            bad |= c == r
        cols[sel] = c
        if not bad.any():
            break
        cols[sel[bad]] = draw(rng, r[bad])
        bad_rows = np.unique(r[bad])
        sel = _concat_ranges(rowptr[bad_rows], deg[bad_rows])
    else:  # pragma: no cover - would need a pathological degree / K ratio
        raise RuntimeError("could not draw distinct columns")
    return rowptr, cols


def _uniform_cols(K: int):
    def draw(rng, rows):
        return rng.integers(0, K, size=rows.size, dtype=np.int64)
    return draw


def _gen_tiny(M: int, rng_s, rng_v):
    deg = rng_s.poisson(8.0, size=M).astype(np.int64)
    deg = np.minimum(deg, M)
    n_empty = max(1, M // 100)
    empty = rng_s.choice(M, size=n_empty, replace=False)
    deg[empty] = 0
    rowptr, col = _distinct_columns(rng_s, deg, M, _uniform_cols(M))
    val = rng_v.random(col.size, dtype=np.float32)
    return rowptr, col, val


def _gen_road(M: int, rng_s, rng_v):
    deg = rng_s.poisson(3.0, size=M).astype(np.int64)
    deg = np.minimum(deg, 256)

    def draw(rng, rows):
        k = rng.integers(0, 512, size=rows.size, dtype=np.int64)
        off = np.where(k < 256, k - 256, k - 255)          # [-256,-1] U [1,256]
        return np.clip(rows + off, 0, M - 1)

    rowptr, col = _distinct_columns(rng_s, deg, M, draw, forbid_self=True)
    return rowptr, col, None


def _powerlaw_degrees(rng, M: int, alpha=2.1, dmin=1, dmax=50_000, target=25.0):
    d = np.arange(dmin, dmax + 1, dtype=np.float64)
    pmf = d ** (-alpha)
    cdf = np.cumsum(pmf)
    cdf /= cdf[-1]
    u = rng.random(M)
    raw = np.searchsorted(cdf, u, side="right").astype(np.int64) + dmin
    raw = np.minimum(raw, dmax)

    def scaled(s):
        return np.clip(np.rint(s * raw), dmin, dmax).astype(np.int64)

    lo, hi = 0.5, 200.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        m = scaled(mid).mean()
        if abs(m - target) <= 0.1:
            return scaled(mid)
        if m < target:
            lo = mid
        else:
            hi = mid
    return scaled(0.5 * (lo + hi))


def _gen_powerlaw(M: int, rng_s, rng_v):
    dmax = min(50_000, M)
    deg = _powerlaw_degrees(rng_s, M, dmax=dmax)
    rowptr, col = _distinct_columns(rng_s, deg, M, _uniform_cols(M))
    rows = np.repeat(np.arange(M, dtype=np.int64), deg)
    degf = deg.astype(np.float64)
    val = (1.0 / np.sqrt(degf[rows] * degf[col])).astype(np.float32)
    return rowptr, col, val


def _gen_diffusion(M: int, rng_s, rng_v, k=10, sigma=500.0):
    deg = np.full(M, min(k, M), dtype=np.int64)

    def draw(rng, rows):
        z = rng.standard_normal(rows.size)
        return np.mod(rows + np.rint(sigma * z).astype(np.int64), M)

    rowptr, col = _distinct_columns(rng_s, deg, M, draw)
    return rowptr, col, None


def _gen_community(M: int, rng_s, rng_v, size=256, p=0.1, n_inter=2):
    starts = np.arange(0, M, size, dtype=np.int64)
    rows_l, cols_l = [], []
    # intra-community Bernoulli(p) edges, self included, drawn community by community
    for c0 in starts:
        s = int(min(size, M - c0))
        mask = rng_s.random((s, s)) < p
        r, c = np.nonzero(mask)
        rows_l.append(r.astype(np.int64) + c0)
        cols_l.append(c.astype(np.int64) + c0)
    rows_in = np.concatenate(rows_l)
    cols_in = np.concatenate(cols_l)
    # n_inter distinct uniform neighbours outside the row's own community
    rows_out = np.repeat(np.arange(M, dtype=np.int64), n_inter)
    cstart = (rows_out // size) * size
    csize = np.minimum(size, M - cstart)

    def draw_out(idx):
        j = (rng_s.random(idx.size) * (M - csize[idx])).astype(np.int64)
        return np.where(j >= cstart[idx], j + csize[idx], j)

    cols_out = draw_out(np.arange(rows_out.size))
    for _ in range(1000):
        pair = cols_out.reshape(M, n_inter)
        dup = np.zeros_like(pair, dtype=bool)
        for a in range(1, n_inter):
            dup[:, a] = (pair[:, :a] == pair[:, a:a + 1]).any(axis=1)
        dup = dup.reshape(-1)
        if not dup.any():
            break
        idx = np.nonzero(dup)[0]
        cols_out[idx] = draw_out(idx)
    rows = np.concatenate([rows_in, rows_out])
    cols = np.concatenate([cols_in, cols_out])
    order = np.argsort(rows * np.int64(M) + cols, kind="stable")
    rows = rows[order]
    cols = cols[order]
    deg = np.bincount(rows, minlength=M).astype(np.int64)
    rowptr = _rowptr_from_deg(deg)
    val = rng_v.random(cols.size, dtype=np.float32)
    return rowptr, cols, val


def _gen_mixed(M: int, rng_s, rng_v):
    """Rows [0, M/3): road-like band; [M/3, 2M/3): 256-node communities
    (columns in that part); the rest: power-law degrees (mean 25) with
    uniform columns over all M.  Weights U[0, 1)."""
    m1 = M // 3
    m2 = M // 3
    m3 = M - m1 - m2
    rp1, c1, _ = _gen_road(m1, rng_s, rng_v)
    rp2, c2, _ = _gen_community(m2, rng_s, rng_v)
    deg3 = _powerlaw_degrees(rng_s, m3, dmax=min(50_000, M))
    rp3, c3 = _distinct_columns(rng_s, deg3, M, _uniform_cols(M))
    rowptr = np.concatenate([rp1, rp1[-1] + rp2[1:], rp1[-1] + rp2[-1] + rp3[1:]]).astype(np.int64)
    col = np.concatenate([c1, c2 + m1, c3]).astype(np.int64)
    val = rng_v.random(col.size, dtype=np.float32)
    return rowptr, col, val


def _gen_knn(M: int, rng_s, rng_v):
    g = knn_line(M, 10)
    return g.rowptr, g.col, None


_GENERATORS = {
    "tiny": _gen_tiny,
    "road": _gen_road,
    "powerlaw": _gen_powerlaw,
    "diffusion": _gen_diffusion,
    "community": _gen_community,
    "mixed": _gen_mixed,
    "knn": _gen_knn,
}


def make_graph(name: str, M: Optional[int] = None, seed: Optional[int] = None) -> Graph:
    """Graph of regime ``name``; ``M`` overrides the row count (M = K)."""
    cfg = CONFIGS[name]
    M = int(cfg["M"] if M is None else M)
    seed = int(cfg["seed"] if seed is None else seed)
    rng_s, rng_v, _ = _streams(seed)
    rowptr, col, val = _GENERATORS[name](M, rng_s, rng_v)
    return Graph(name=name, M=M, K=M, rowptr=rowptr, col=col, val=val)


def make_features(name: str, K: int, N: int, seed: Optional[int] = None) -> np.ndarray:
    """Dense operand B [K, N] fp32: U[0,1) for diffusion, N(0,1) otherwise."""
    cfg = CONFIGS[name]
    seed = int(cfg["seed"] if seed is None else seed)
    _, _, rng_f = _streams(seed)
    if name == "diffusion":
        return rng_f.random((K, N), dtype=np.float32)
    return rng_f.standard_normal((K, N), dtype=np.float32)


def make(name: str, M: Optional[int] = None, N: Optional[int] = None,
         seed: Optional[int] = None) -> Workload:
    cfg = CONFIGS[name]
    g = make_graph(name, M=M, seed=seed)
    N = int(cfg["N"] if N is None else N)
    B = make_features(name, g.K, N, seed=seed)
    return Workload(graph=g, N=N, B=B, reduces=tuple(cfg["reduces"]))


# ---------------------------------------------------------------------------
# small irregular CSR matrices for edge cases
# ---------------------------------------------------------------------------

def csr_from_pairs(M: int, rows: np.ndarray, cols: np.ndarray):
    """Stable grouping of (row, col) pairs by row; within-row order is kept."""
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    order = np.argsort(rows, kind="stable")
    deg = np.bincount(rows, minlength=M).astype(np.int64)
    return _rowptr_from_deg(deg), cols[order], order


def random_csr(rng: np.random.Generator, M: int, K: int, mean_deg: float = 4.0,
               empty_frac: float = 0.1, dup_frac: float = 0.0, shuffle_rows: bool = False,
               zero_frac: float = 0.0, weighted: bool = True, heavy_rows: int = 0,
               heavy_deg: int = 0) -> Graph:
    """Irregular CSR: Poisson degrees, forced empty rows, optional duplicate
    entries, unsorted columns, explicit stored zeros and a few very long rows."""
    deg = rng.poisson(mean_deg, size=M).astype(np.int64)
    if M and empty_frac > 0:
        n_empty = int(round(empty_frac * M))
        deg[rng.choice(M, size=min(n_empty, M), replace=False)] = 0
    if heavy_rows and M:
        hr = rng.choice(M, size=min(heavy_rows, M), replace=False)
        deg[hr] = heavy_deg
    if K == 0:
        deg[:] = 0
    rowptr = _rowptr_from_deg(deg)
    nnz = int(rowptr[-1])
    col = rng.integers(0, max(K, 1), size=nnz, dtype=np.int64)
    if dup_frac > 0 and nnz > 1:
        # copy the previous entry's column onto a fraction of entries (same row only)
        rows = np.repeat(np.arange(M, dtype=np.int64), deg)
        pick = np.nonzero((rng.random(nnz) < dup_frac))[0]
        pick = pick[pick > 0]
        pick = pick[rows[pick] == rows[pick - 1]]
        col[pick] = col[pick - 1]
    if not shuffle_rows:
        for i in range(M):
            a, b = rowptr[i], rowptr[i + 1]
            if b - a > 1:
                col[a:b] = np.sort(col[a:b], kind="stable")
    val = None
    if weighted:
        val = rng.random(nnz, dtype=np.float32)
        if zero_frac > 0:
            val[rng.random(nnz) < zero_frac] = 0.0
    return Graph(name="random", M=M, K=K, rowptr=rowptr, col=col, val=val)


def block_csr(rng: np.random.Generator, M: int, K: int, in_deg: float = 12.0, off_deg: float = 2.0,
              empty_frac: float = 0.05, weighted: bool = True, block: int = 256) -> Graph:
    """Block-structured CSR: row i draws Poisson(in_deg) columns with
    replacement (so duplicates occur) from its own aligned block of `block`
    columns [block*(i//block), ...) clipped to K, plus Poisson(off_deg) columns
    uniform over [0, K); each row's entries are shuffled (unsorted) and a
    fraction of rows is forced empty."""
    d_in = rng.poisson(in_deg, size=M).astype(np.int64)
    d_off = rng.poisson(off_deg, size=M).astype(np.int64)
    lo = (np.arange(M, dtype=np.int64) // block) * block
    hi = np.minimum(lo + block, K)
    d_in[lo >= hi] = 0                      # block entirely beyond K
    if M and empty_frac > 0:
        e = rng.choice(M, size=min(int(round(empty_frac * M)), M), replace=False)
        d_in[e] = 0
        d_off[e] = 0
    if K == 0:
        d_off[:] = 0
    deg = d_in + d_off
    rowptr = _rowptr_from_deg(deg)
    nnz = int(rowptr[-1])
    col = np.empty(nnz, dtype=np.int64)
    rows = np.repeat(np.arange(M, dtype=np.int64), deg)
    pos = np.arange(nnz, dtype=np.int64) - rowptr[rows]
    inside = pos < d_in[rows]
    span = (hi - lo)[rows]
    col[inside] = lo[rows][inside] + (rng.random(int(inside.sum())) * span[inside]).astype(np.int64)
    col[~inside] = rng.integers(0, max(K, 1), size=int((~inside).sum()), dtype=np.int64)
    for i in range(M):                       # shuffle within each row
        a, b = rowptr[i], rowptr[i + 1]
        if b - a > 1:
            col[a:b] = col[a:b][rng.permutation(b - a)]
    val = rng.random(nnz, dtype=np.float32) if weighted else None
    return Graph(name="block", M=M, K=K, rowptr=rowptr, col=col, val=val)


def knn_line(M: int, k: int = 10) -> Graph:
    """k-nearest-neighbour graph of M points on a line: row i holds the k/2
    nearest points on each side (i - k/2 .. i + k/2 without i, clipped to
    [0, M)), ascending, unweighted.  Adjacent rows share all but a few
    neighbours: the locality that vectorized blocking exploits."""
    h = k // 2
    i = np.arange(M, dtype=np.int64)
    offs = np.concatenate([np.arange(-h, 0), np.arange(1, h + 1)]).astype(np.int64)
    cand = i[:, None] + offs[None, :]
    keep = (cand >= 0) & (cand < M)
    deg = keep.sum(axis=1).astype(np.int64)
    return Graph(name="knn", M=M, K=M, rowptr=_rowptr_from_deg(deg), col=cand[keep], val=None)


def relabel(g: Graph, seed: int) -> Graph:
    """The same graph under uniformly random node ids (square graphs): node u
    becomes pi[u] for a seeded permutation pi; every row keeps its entries in
    their stored order.  Hides the locality of the original numbering."""
    assert g.M == g.K
    rng = np.random.default_rng(seed)
    pi = rng.permutation(g.M).astype(np.int64)
    inv = np.empty_like(pi)
    inv[pi] = np.arange(g.M)
    deg = g.degrees()[inv]                      # new row r is old row inv[r]
    rowptr = _rowptr_from_deg(deg)
    src = _concat_ranges(g.rowptr[:-1][inv], deg)
    col = pi[g.col[src]]
    val = None if g.val is None else g.val[src]
    return Graph(name=g.name + "-relabelled", M=g.M, K=g.K, rowptr=rowptr, col=col, val=val)


# --- Graphs at the library's index limits -------------------------------------
#
# Too large to build on the host, these are given by formulas on integer
# arrays: a test evaluates them on the device (torch tensors) to build the
# graph and on the host (numpy arrays) to rebuild any row it samples.  Only
# the integer operators *, +, % and // are used, which both libraries apply
# elementwise with the same int64 results (no product exceeds 2^63).

HASH_MUL = 2654435761        # Knuth's multiplicative hashing constant, 2^32 / golden ratio


def hashed_cols(p, K: int):
    """Column of the entry at position p (0 <= p < 2^31): (p * 2654435761 + 7)
    mod K, spread over [0, K) with no order within a row."""
    return (p * HASH_MUL + 7) % K


def small_int_features(j):
    """Feature of B row j, an integer in [-1000, 1000] (exact in fp32):
    (j * 40503) mod 2001 - 1000."""
    return (j * 40503) % 2001 - 1000


def alternating_rowptr(i):
    """rowptr of the graph whose odd rows hold one entry and even rows none:
    rowptr[i] = i // 2."""
    return i // 2


def limit_degrees(M: int, nnz: int, n_heavy: int, giant: int) -> np.ndarray:
    """Degrees of M rows summing to exactly nnz: light row i holds
    (i * 7919) mod 701 entries, row M - 1 holds `giant` entries, and n_heavy
    rows spread evenly over [0, M - 1) share the remainder (the first of them
    takes what does not divide evenly)."""
    deg = (np.arange(M, dtype=np.int64) * 7919) % 701
    heavy = np.linspace(0, M - 2, n_heavy).astype(np.int64)
    deg[heavy] = 0
    deg[M - 1] = giant
    rest = nnz - int(deg.sum())
    assert rest > 0, "light rows and the giant row already exceed nnz"
    deg[heavy] = rest // n_heavy
    deg[heavy[0]] += rest - (rest // n_heavy) * n_heavy
    return deg

"""The allocation-free edge-list sort (spmm_coo_to_csr_noalloc) through the C
ABI: its output must equal spmm_coo_to_csr's bit for bit, on two calls in a
row (the second smaller, so stale workspace contents from the first would
show), and it must allocate nothing on the library's ledger."""
import ctypes

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gnn_sparse_dense_amd as G
    from tests.gpu_helpers import DEV, log

MAX_EDGES = 1 << 20


def _edges(seed, E, M, K, weighted=True):
    rng = np.random.default_rng(seed)
    row = torch.from_numpy(rng.integers(0, M, E).astype(np.int64)).to(DEV)
    col = torch.from_numpy(rng.integers(0, K, E).astype(np.int64)).to(DEV)
    val = torch.from_numpy(rng.random(E, dtype=np.float32)).to(DEV) if weighted else None
    return row, col, val


def _noalloc(row, col, val, M, K):
    E = row.numel()
    rp = torch.full((M + 1,), -7, dtype=torch.int64, device=DEV)
    c = torch.full((max(E, 1),), -7, dtype=torch.int64, device=DEV)[:E]
    v = None if val is None else torch.full((max(E, 1),), float("nan"), dtype=torch.float32, device=DEV)[:E]
    lib = G.lib()
    st = lib.spmm_coo_to_csr_noalloc(G._addr(row), G._addr(col), G._addr(val), E, M, K, G._addr(rp), G._addr(c),
                                     G._addr(v))
    torch.cuda.synchronize()
    return st, rp, c, v


@pytest.mark.parametrize("weighted", [True, False])
def test_noalloc_matches_allocating_sort(weighted):
    base = G.spmm_mem_stats()["in_use"]
    for i, (E, M, K) in enumerate(((MAX_EDGES, 50000, 40000), (30001, 3000, 2000), (0, 17, 5))):
        log(f"no-alloc edge sort: call {i}, E={E} M={M} K={K} weighted={weighted}")
        row, col, val = _edges(100 + i, E, M, K, weighted)
        st, rp, c, v = _noalloc(row, col, val, M, K)
        assert st == G.SPMM_OK, G.spmm_last_error()
        assert G.spmm_mem_stats()["in_use"] == base
        rp2, c2, v2 = G.spmm_coo_to_csr(row, col, val, M, K)
        torch.cuda.synchronize()
        assert torch.equal(rp, rp2) and torch.equal(c, c2)
        if weighted:
            assert torch.equal(v.view(torch.int32), v2.view(torch.int32))


def test_noalloc_errors():
    row, col, val = _edges(7, 100, 10, 10)
    col[5] = 10                                          # column outside [0, K)
    st, *_ = _noalloc(row, col, val, 10, 10)
    assert st == G.SPMM_E_BAD_CSR and "edge 5" in G.spmm_last_error()[1]
    # beyond the workspace: rejected on the host before any launch
    lib = G.lib()
    big = torch.zeros(1, dtype=torch.int64, device=DEV)
    st = lib.spmm_coo_to_csr_noalloc(G._addr(big), G._addr(big), None, MAX_EDGES + 1, 1, 1, G._addr(big),
                                     G._addr(big), None)
    assert st == G.SPMM_E_UNSUPPORTED and "at most" in G.spmm_last_error()[1]
    # a good call afterwards still matches
    row, col, val = _edges(8, 5000, 300, 300)
    st, rp, c, v = _noalloc(row, col, val, 300, 300)
    assert st == G.SPMM_OK
    rp2, c2, v2 = G.spmm_coo_to_csr(row, col, val, 300, 300)
    assert torch.equal(rp, rp2) and torch.equal(c, c2) and torch.equal(v, v2)

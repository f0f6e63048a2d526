"""Seeded synthetic inputs for CSR sparse x dense products (GNN neighbour aggregation).

This module only builds inputs: graph structure (CSR), edge weights and the dense
feature matrix.  It holds none of the product's arithmetic, so both the HIP path
and the CPU oracle can be fed from it without sharing any computation.
"""
from .graphs import (  # noqa: F401
    CONFIGS,
    Graph,
    Workload,
    make,
    make_graph,
    make_features,
    random_csr,
    block_csr,
    knn_line,
    relabel,
    csr_from_pairs,
    hashed_cols,
    small_int_features,
    alternating_rowptr,
    limit_degrees,
)

"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
and compare with the CPU oracle at the tolerances the product states.

Tolerances:
* sum / mean: |GPU - oracle| <= 1e-5 * sum_p |a_p * b_p| + 1e-6 per element,
  with the sum of magnitudes from the oracle in float64;
* max values and argmax: bit-exact;
* rows the GPU walks whole (not split): additionally bit-exact against the
  oracle's fused-multiply-add mode, since both then accumulate in stored
  order with one rounding per entry.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import gnn_sparse_dense_amd as G

DEV = torch.device("cuda:0")
REL_TOL = 1e-5
ABS_TOL = 1e-6


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(g, B=None):
    rowptr = torch.from_numpy(np.ascontiguousarray(g.rowptr)).to(DEV)
    col = torch.from_numpy(np.ascontiguousarray(g.col)).to(DEV)
    val = None if g.val is None else torch.from_numpy(np.ascontiguousarray(g.val)).to(DEV)
    Bd = None if B is None else torch.from_numpy(np.ascontiguousarray(B)).to(DEV)
    return rowptr, col, val, Bd


def make_plan(g, options=()):
    rowptr, col, val, _ = to_dev(g)
    plan = G.spmm_plan_create(rowptr, col, val, g.M, g.K)
    for opt, v in options:
        G.spmm_plan_set_option(plan, opt, v)
    return plan


def gpu_run(plan, M, Bd, reduce, poison=True, stream=None):
    """Run once and return host copies (C, argmax or None)."""
    N = Bd.shape[1]
    C = torch.empty((M, N), dtype=torch.float32, device=DEV)
    arg = torch.empty((M, N), dtype=torch.int64, device=DEV) if reduce == "max" else None
    if poison:
        C.fill_(float("nan"))
        if arg is not None:
            arg.fill_(0x7F7F7F7F7F7F7F7F)
    G.spmm_run(plan, Bd, C, arg, N, reduce, stream)
    torch.cuda.synchronize()
    return C.cpu().numpy(), (None if arg is None else arg.cpu().numpy())


def check(orc, g, B, reduce, C, arg, rows=None, exact_rows=None, what=""):
    """Compare GPU output (for `rows`, or all rows) with the oracle."""
    if reduce == "max":
        refC, refA = orc.spmm(g.rowptr, g.col, g.val, g.M, g.K, B, "max", rows=rows)
        bad = C.view(np.uint32) != refC.view(np.uint32)
        assert not bad.any(), f"{what}: {int(bad.sum())} max values differ"
        if arg is not None:
            badA = arg != refA
            assert not badA.any(), f"{what}: {int(badA.sum())} argmax entries differ"
        return
    ref = orc.spmm(g.rowptr, g.col, g.val, g.M, g.K, B, reduce, rows=rows)
    S = orc.sumabs(g.rowptr, g.col, g.val, g.M, B, rows=rows)
    err = np.abs(C.astype(np.float64) - ref.astype(np.float64))
    bad = ~(err <= REL_TOL * S + ABS_TOL)
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outside tolerance, "
                           f"max err {np.nanmax(err):.3e}")
    if exact_rows is not None and len(exact_rows):
        ref_f = orc.spmm(g.rowptr, g.col, g.val, g.M, g.K, B, reduce, fused=True, rows=rows)
        sel = exact_rows
        diff = C[sel].view(np.uint32) != ref_f[sel].view(np.uint32)
        assert not diff.any(), f"{what}: {int(diff.sum())} whole-row results differ from the fused oracle"

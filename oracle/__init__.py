"""ctypes front end of the CPU oracle (oracle/spmm_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the package smoke check and by
the benchmark's CPU-baseline leg.  The product path never imports it.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

SUM, MEAN, MAX = 0, 1, 2
REDUCE = {"sum": SUM, "mean": MEAN, "max": MAX}

_p = ctypes.c_void_p
_i64 = ctypes.c_int64


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    def __init__(self, path: str = LIB_PATH):
        if not os.path.exists(path):
            from . import build as _b
            _b.build(out=path)
        lib = ctypes.CDLL(path)
        lib.oracle_spmm.argtypes = [_p, _p, _p, _i64, _i64, _p, _i64, ctypes.c_int,
                                    ctypes.c_int, _p, _i64, _p, _p]
        lib.oracle_spmm.restype = ctypes.c_int
        lib.oracle_sumabs.argtypes = [_p, _p, _p, _i64, _p, _i64, _p, _i64, _p]
        lib.oracle_sumabs.restype = ctypes.c_int
        lib.oracle_validate.argtypes = [_p, _p, _i64, _i64]
        lib.oracle_validate.restype = _i64
        lib.oracle_descriptors.argtypes = [_p, _i64, _p, _p]
        lib.oracle_descriptors.restype = None
        lib.oracle_partition.argtypes = [_p, _i64, _i64, _i64, _p, _p, _p, _i64, _p, _i64, _p]
        lib.oracle_partition.restype = ctypes.c_int
        lib.oracle_mac_gap.argtypes = [_i64, _i64, _i64]
        lib.oracle_mac_gap.restype = _i64
        lib.oracle_coo_to_csr.argtypes = [_p, _p, _p, _i64, _i64, _i64, _p, _p, _p]
        lib.oracle_coo_to_csr.restype = _i64
        lib.oracle_transpose.argtypes = [_p, _p, _p, _i64, _i64, ctypes.c_int, _p, _p, _p]
        lib.oracle_transpose.restype = None
        lib.oracle_max_backward.argtypes = [_p, _p, _i64, _i64, _i64, _p]
        lib.oracle_max_backward.restype = ctypes.c_int
        lib.oracle_features.argtypes = [_p, _p, _i64, _i64, _i64, _p, _p]
        lib.oracle_features.restype = ctypes.c_int
        lib.oracle_rcm.argtypes = [_p, _p, _i64, _p]
        lib.oracle_rcm.restype = ctypes.c_int
        lib.oracle_permute.argtypes = [_p, _p, _p, _i64, _p, _p, _p, _p]
        lib.oracle_permute.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    @staticmethod
    def _csr(rowptr, col, val):
        rowptr = np.ascontiguousarray(rowptr, dtype=np.int64)
        col = np.ascontiguousarray(col, dtype=np.int64)
        val = None if val is None else np.ascontiguousarray(val, dtype=np.float32)
        return rowptr, col, val

    def spmm(self, rowptr, col, val, M, K, B, reduce="sum", fused=False, rows=None):
        """Returns C [nrows, N] fp32 and, for max, argmax [nrows, N] int64."""
        rowptr, col, val = self._csr(rowptr, col, val)
        B = np.ascontiguousarray(B, dtype=np.float32)
        N = B.shape[1]
        red = REDUCE[reduce] if isinstance(reduce, str) else int(reduce)
        rows_a = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
        nrows = M if rows_a is None else rows_a.size
        C = np.empty((nrows, N), dtype=np.float32)
        arg = np.empty((nrows, N), dtype=np.int64) if red == MAX else None
        rc = self.lib.oracle_spmm(_ptr(rowptr), _ptr(col), _ptr(val), M, K, _ptr(B), N, red,
                                  int(bool(fused)), _ptr(rows_a), nrows, _ptr(C), _ptr(arg))
        if rc != 0:
            raise ValueError("oracle_spmm rejected its arguments")
        return (C, arg) if red == MAX else C

    def sumabs(self, rowptr, col, val, M, B, rows=None):
        rowptr, col, val = self._csr(rowptr, col, val)
        B = np.ascontiguousarray(B, dtype=np.float32)
        N = B.shape[1]
        rows_a = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
        nrows = M if rows_a is None else rows_a.size
        S = np.empty((nrows, N), dtype=np.float64)
        rc = self.lib.oracle_sumabs(_ptr(rowptr), _ptr(col), _ptr(val), M, _ptr(B), N,
                                    _ptr(rows_a), nrows, _ptr(S))
        if rc != 0:
            raise ValueError("oracle_sumabs rejected its arguments")
        return S

    def validate(self, rowptr, col, M, K) -> int:
        rowptr, col, _ = self._csr(rowptr, col, None)
        return int(self.lib.oracle_validate(_ptr(rowptr), _ptr(col), M, K))

    def descriptors(self, rowptr, M):
        rowptr = np.ascontiguousarray(rowptr, dtype=np.int64)
        ints = np.zeros(3, dtype=np.int64)
        dbl = np.zeros(2, dtype=np.float64)
        self.lib.oracle_descriptors(_ptr(rowptr), M, _ptr(ints), _ptr(dbl))
        return dict(nnz=int(ints[0]), dmax=int(ints[1]), n_empty=int(ints[2]),
                    mean=float(dbl[0]), cv=float(dbl[1]))

    def partition(self, rowptr, M, T, L):
        rowptr = np.ascontiguousarray(rowptr, dtype=np.int64)
        counts = np.zeros(3, dtype=np.int64)
        z = np.zeros(0, dtype=np.int64)
        rc = self.lib.oracle_partition(_ptr(rowptr), M, T, L, _ptr(z), _ptr(z), _ptr(z), 0,
                                       _ptr(z), 0, _ptr(counts))
        if rc != 0:
            raise ValueError("oracle_partition rejected its arguments")
        n_seg, n_light = int(counts[1]), int(counts[2])
        sr = np.empty(n_seg, np.int64)
        sb = np.empty(n_seg, np.int64)
        se = np.empty(n_seg, np.int64)
        light = np.empty(n_light, np.int64)
        self.lib.oracle_partition(_ptr(rowptr), M, T, L, _ptr(sr), _ptr(sb), _ptr(se), n_seg,
                                  _ptr(light), n_light, _ptr(counts))
        return dict(n_heavy=int(counts[0]), seg_row=sr, seg_begin=sb, seg_end=se, light=light)

    def mac_gap(self, dim, F, omega) -> int:
        return int(self.lib.oracle_mac_gap(dim, F, omega))

    def coo_to_csr(self, row, col, val, M, K):
        """(rowptr, col, val) of the stable row-grouping of an edge list; raises
        ValueError naming the first bad edge."""
        row = np.ascontiguousarray(row, dtype=np.int64)
        col = np.ascontiguousarray(col, dtype=np.int64)
        val = None if val is None else np.ascontiguousarray(val, dtype=np.float32)
        E = row.size
        rp = np.empty(M + 1, np.int64)
        co = np.empty(E, np.int64)
        vo = None if val is None else np.empty(E, np.float32)
        bad = self.lib.oracle_coo_to_csr(_ptr(row), _ptr(col), _ptr(val), E, M, K, _ptr(rp), _ptr(co), _ptr(vo))
        if bad != -1:
            raise ValueError(f"bad edge {bad}")
        return rp, co, vo

    def transpose(self, rowptr, col, val, M, K, scale=False):
        rowptr, col, val = self._csr(rowptr, col, val)
        nnz = int(rowptr[M])
        rt = np.empty(K + 1, np.int64)
        ct = np.empty(nnz, np.int64)
        vt = np.empty(nnz, np.float32)
        self.lib.oracle_transpose(_ptr(rowptr), _ptr(col), _ptr(val), M, K, int(bool(scale)), _ptr(rt),
                                  _ptr(ct), _ptr(vt))
        return rt, ct, vt

    def max_backward(self, argmax, dC, M, K):
        argmax = np.ascontiguousarray(argmax, dtype=np.int64)
        dC = np.ascontiguousarray(dC, dtype=np.float32)
        N = dC.shape[1]
        dB = np.empty((K, N), np.float32)
        if self.lib.oracle_max_backward(_ptr(argmax), _ptr(dC), M, K, N, _ptr(dB)) != 0:
            raise ValueError("argmax entry outside [-1, K)")
        return dB

    def features(self, rowptr, col, M, K, V=2):
        """ParamSpMM Table 3 features (see oracle_features)."""
        rowptr, col, _ = self._csr(rowptr, col, None)
        ints = np.zeros(7, np.int64)
        dbl = np.zeros(8, np.float64)
        if self.lib.oracle_features(_ptr(rowptr), _ptr(col), M, K, V, _ptr(ints), _ptr(dbl)) != 0:
            raise ValueError("oracle_features rejected its arguments")
        names_i = ("n", "n_nonempty", "nnz", "dmax", "max_bandwidth", "nnz_distinct", "nnz_vectors")
        names_d = ("delta", "mean_deg", "mean_deg_nonempty", "cv_deg", "cv_deg_nonempty", "density",
                   "mean_bandwidth", "padding_ratio")
        out = {k: int(v) for k, v in zip(names_i, ints)}
        out.update({k: float(v) for k, v in zip(names_d, dbl)})
        out["V"] = int(V)
        return out

    def rcm(self, rowptr, col, M):
        """Reverse Cuthill-McKee permutation (perm[i] = node at position i)."""
        rowptr, col, _ = self._csr(rowptr, col, None)
        perm = np.empty(M, np.int64)
        if self.lib.oracle_rcm(_ptr(rowptr), _ptr(col), M, _ptr(perm)) != 0:
            raise MemoryError("oracle_rcm")
        return perm

    def permute(self, rowptr, col, val, M, perm):
        """CSR of P A P^T (see oracle_permute)."""
        rowptr, col, val = self._csr(rowptr, col, val)
        perm = np.ascontiguousarray(perm, dtype=np.int64)
        nnz = int(rowptr[M])
        rp = np.empty(M + 1, np.int64)
        cp = np.empty(nnz, np.int64)
        vp = None if val is None else np.empty(nnz, np.float32)
        if self.lib.oracle_permute(_ptr(rowptr), _ptr(col), _ptr(val), M, _ptr(perm), _ptr(rp), _ptr(cp),
                                   _ptr(vp)) != 0:
            raise ValueError("perm is not a permutation of [0, M)")
        return rp, cp, vp


_default: Optional[Oracle] = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default

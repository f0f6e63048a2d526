"""Python binding of the gfx950 CSR SpMM library (include/spmm.h).

Argument marshalling only: every step of the product runs in the HIP library
libgnn_spmm.so next to this file.  PyTorch supplies device memory and the
current stream.  Importing this package fails loudly when the library has not
been built; there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgnn_spmm.so")

SPMM_SUM, SPMM_MEAN, SPMM_MAX = 0, 1, 2
REDUCE = {"sum": SPMM_SUM, "mean": SPMM_MEAN, "max": SPMM_MAX}

SPMM_OK = 0
SPMM_E_INVALID_ARG = -1
SPMM_E_BAD_CSR = -2
SPMM_E_OOM = -3
SPMM_E_HIP = -4
SPMM_E_UNSUPPORTED = -5

SPMM_OPT_SPLIT_T = 1
SPMM_OPT_SPLIT_L = 2
SPMM_OPT_SPLIT_MODE = 3
SPMM_OPT_LANES = 4
SPMM_OPT_COARSEN = 5
SPMM_OPT_VEC = 6
SPMM_OPT_XCD_REMAP = 7
SPMM_OPT_NT_STORE = 8
SPMM_OPT_TILES = 9
SPMM_OPT_WINDOW = 10
SPMM_OPT_MFMA = 11
SPMM_OPT_VBLOCK = 12
SPMM_OPT_BALANCE = 13
SPMM_OPT_PIECE_ORDER = 14
SPMM_OPT_MEM_LIMIT = 15
SPMM_OPT_SPLIT_FUSED = 16

SPMM_REORDER_RCM = 1

EXPORTED = (
    "spmm_plan_create", "spmm_run", "spmm_plan_destroy", "spmm_plan_info",
    "spmm_plan_route", "spmm_plan_partition", "spmm_plan_set_option", "spmm_last_error",
    "spmm_coo_to_csr", "spmm_plan_transpose", "spmm_max_backward", "spmm_plan_features",
    "spmm_plan_reorder", "spmm_plan_permute", "spmm_set_mem_limit", "spmm_mem_stats",
    "spmm_coo_to_csr_noalloc",
)


class SpmmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


class _Info(ctypes.Structure):
    _fields_ = [
        ("M", ctypes.c_int64), ("K", ctypes.c_int64), ("nnz", ctypes.c_int64),
        ("dmax", ctypes.c_int64), ("n_empty", ctypes.c_int64),
        ("mean_deg", ctypes.c_double), ("cv_deg", ctypes.c_double),
        ("split_T", ctypes.c_int64), ("split_L", ctypes.c_int64),
        ("n_heavy", ctypes.c_int64), ("n_seg", ctypes.c_int64),
        ("split_ratio", ctypes.c_double),
        ("has_val", ctypes.c_int32), ("index_bits", ctypes.c_int32),
        ("plan_ms", ctypes.c_double),
        ("route_N", ctypes.c_int64),
        ("route_lanes", ctypes.c_int32), ("route_vec", ctypes.c_int32),
        ("route_coarsen", ctypes.c_int32), ("route_rows_per_wave", ctypes.c_int32),
        ("route_slices", ctypes.c_int32), ("route_xcd_remap", ctypes.c_int32),
        ("route_nt_store", ctypes.c_int32), ("route_split", ctypes.c_int32),
        ("tiles", ctypes.c_int32), ("tile_cap", ctypes.c_int32),
        ("route_tiled", ctypes.c_int32), ("route_window", ctypes.c_int32),
        ("win_frac", ctypes.c_double), ("tile_overflow", ctypes.c_int64),
        ("mfma_resid_nnz", ctypes.c_int64),
        ("mfma_tiles", ctypes.c_int32), ("route_mfma", ctypes.c_int32),
        ("pair_vectors", ctypes.c_int64), ("pair_padding", ctypes.c_double),
        ("pairs_built", ctypes.c_int32), ("route_pairs", ctypes.c_int32),
        ("merge_segments", ctypes.c_int64), ("route_merge", ctypes.c_int32), ("piece_order", ctypes.c_int32),
        ("generation", ctypes.c_int64), ("device_bytes", ctypes.c_int64), ("mem_limit", ctypes.c_int64),
        ("route_fused_split", ctypes.c_int32),
    ]


class _MemStats(ctypes.Structure):
    _fields_ = [
        ("in_use", ctypes.c_int64), ("last_call_peak", ctypes.c_int64),
        ("last_call_allocs", ctypes.c_int64), ("thread_limit", ctypes.c_int64),
    ]


class _Features(ctypes.Structure):
    _fields_ = [
        ("n", ctypes.c_int64), ("n_nonempty", ctypes.c_int64), ("nnz", ctypes.c_int64),
        ("dmax", ctypes.c_int64),
        ("delta", ctypes.c_double), ("mean_deg", ctypes.c_double), ("mean_deg_nonempty", ctypes.c_double),
        ("cv_deg", ctypes.c_double), ("cv_deg_nonempty", ctypes.c_double), ("density", ctypes.c_double),
        ("mean_bandwidth", ctypes.c_double), ("max_bandwidth", ctypes.c_int64),
        ("V", ctypes.c_int64), ("nnz_distinct", ctypes.c_int64), ("nnz_vectors", ctypes.c_int64),
        ("padding_ratio", ctypes.c_double), ("split_ratio", ctypes.c_double), ("win_frac", ctypes.c_double),
    ]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(LIB_PATH)
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.spmm_plan_create.argtypes = [p, p, p, i64, i64]
    lib.spmm_plan_create.restype = p
    lib.spmm_run.argtypes = [p, p, p, p, i64, i32, p]
    lib.spmm_run.restype = i32
    lib.spmm_plan_destroy.argtypes = [p]
    lib.spmm_plan_destroy.restype = i32
    lib.spmm_plan_info.argtypes = [p, ctypes.POINTER(_Info)]
    lib.spmm_plan_info.restype = i32
    lib.spmm_plan_route.argtypes = [p, i64, i32]
    lib.spmm_plan_route.restype = i32
    lib.spmm_plan_partition.argtypes = [p, p, p, p, i64, p, i64, p]
    lib.spmm_plan_partition.restype = i32
    lib.spmm_plan_set_option.argtypes = [p, i32, i64]
    lib.spmm_plan_set_option.restype = i32
    lib.spmm_plan_features.argtypes = [p, i64, ctypes.POINTER(_Features)]
    lib.spmm_plan_features.restype = i32
    lib.spmm_last_error.argtypes = [ctypes.c_char_p, i64]
    lib.spmm_last_error.restype = i32
    lib.spmm_coo_to_csr.argtypes = [p, p, p, i64, i64, i64, p, p, p]
    lib.spmm_coo_to_csr.restype = i32
    lib.spmm_plan_transpose.argtypes = [p, i32]
    lib.spmm_plan_transpose.restype = p
    lib.spmm_plan_reorder.argtypes = [p, i32, p]
    lib.spmm_plan_reorder.restype = i32
    lib.spmm_plan_permute.argtypes = [p, p]
    lib.spmm_plan_permute.restype = p
    lib.spmm_max_backward.argtypes = [p, p, p, p, i64, p]
    lib.spmm_max_backward.restype = i32
    lib.spmm_coo_to_csr_noalloc.argtypes = [p, p, p, i64, i64, i64, p, p, p]
    lib.spmm_coo_to_csr_noalloc.restype = i32
    lib.spmm_set_mem_limit.argtypes = [i64]
    lib.spmm_set_mem_limit.restype = i32
    lib.spmm_mem_stats.argtypes = [ctypes.POINTER(_MemStats)]
    lib.spmm_mem_stats.restype = i32
    return lib


_lib = _load()


def lib() -> ctypes.CDLL:
    return _lib


def spmm_last_error():
    buf = ctypes.create_string_buffer(512)
    st = _lib.spmm_last_error(buf, 512)
    return st, buf.value.decode(errors="replace")


def _check(status: int):
    if status != SPMM_OK:
        st, msg = spmm_last_error()
        raise SpmmError(status, msg)


def _addr(t) -> Optional[int]:
    """Device address of a tensor (or None), without touching its data."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


_DTYPES: dict = {}


def _dtype_ok(t, dtype: str) -> bool:
    """t.dtype is torch.<dtype> (the torch dtype object is looked up once)."""
    d = _DTYPES.get(dtype)
    if d is None:
        import torch
        d = _DTYPES.setdefault(dtype, getattr(torch, dtype))
    return t.dtype is d


def _current_stream(t) -> int:
    """Raw handle of torch's current stream on the device of tensor t."""
    import torch
    get_raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if get_raw is not None and t is not None and not isinstance(t, int):
        return get_raw(t.get_device())
    return torch.cuda.current_stream().cuda_stream


def _check_matrix(name, t, dtype, rows, cols):
    """A tensor passed by address must be what the library will read or write:
    the C ABI sees only the pointer, so a strided view or a wrong dtype would
    be read as packed row-major data without any error."""
    if t is None or isinstance(t, int):
        return
    if not _dtype_ok(t, dtype):
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (row-major)")
    if t.dim() != 2 or (rows is not None and t.shape[0] != rows) or t.shape[1] != cols:
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected ({rows if rows is not None else 'any'}, {cols})")


def _check_gpu(**tensors):
    for name, t in tensors.items():
        if t is not None and not isinstance(t, int) and not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")


# (M, K) of each live plan handle, so that row counts are checked on the host
# before an address reaches the library (the C ABI cannot see a tensor's size).
_plan_dims: dict = {}


def _dims(plan: int):
    d = _plan_dims.get(plan)
    if d is None:
        info = spmm_plan_info(plan)
        d = (int(info["M"]), int(info["K"]))
        _plan_dims[plan] = d
    return d


def _check_rows(name, t, rows):
    if t is None or isinstance(t, int):
        return
    if t.shape[0] != rows:
        raise ValueError(f"{name} has {t.shape[0]} rows, expected {rows}")


def _check_vector(name, t, dtype, min_len=None, exact_len=None):
    if t is None or isinstance(t, int):
        return
    if not _dtype_ok(t, dtype) or not t.is_contiguous() or t.dim() != 1:
        raise TypeError(f"{name} must be a contiguous 1-D {dtype} tensor")
    if exact_len is not None and t.numel() != exact_len:
        raise ValueError(f"{name} has {t.numel()} elements, expected {exact_len}")
    if min_len is not None and t.numel() < min_len:
        raise ValueError(f"{name} has {t.numel()} elements, fewer than the {min_len} the CSR holds")


def spmm_plan_create(rowptr, col, val, M: int, K: int) -> int:
    """Plan handle for the CSR (rowptr int64 [M+1], col int64 [nnz], val fp32 or None)."""
    M, K = int(M), int(K)
    _check_vector("rowptr", rowptr, "int64", exact_len=M + 1 if M >= 0 else None)
    _check_vector("col", col, "int64")
    _check_vector("val", val, "float32")
    if rowptr is not None and not isinstance(rowptr, int) and M >= 0:
        nnz = int(rowptr[M].item())        # the library reads the same entry
        if nnz >= 0:
            _check_vector("col", col, "int64", min_len=nnz)
            _check_vector("val", val, "float32", min_len=nnz)
    h = _lib.spmm_plan_create(_addr(rowptr), _addr(col), _addr(val), M, K)
    if not h:
        st, msg = spmm_last_error()
        raise SpmmError(st, msg)
    _plan_dims[h] = (M, K)
    return h


def spmm_run(plan: int, B, C, argmax, N: int, reduce, stream=None) -> None:
    """Enqueue C = reduce(A . B) (argmax for 'max' only) on `stream`
    (an int handle, a torch stream, or None for torch's current stream)."""
    red = REDUCE[reduce] if isinstance(reduce, str) else int(reduce)
    _check_matrix("B", B, "float32", None, int(N))
    _check_matrix("C", C, "float32", None, int(N))
    _check_matrix("argmax", argmax, "int64", None if isinstance(C, int) or C is None else C.shape[0], int(N))
    M, K = _dims(plan)
    _check_rows("B", B, K)
    _check_rows("C", C, M)
    _check_rows("argmax", argmax, M)
    _check_gpu(B=B, C=C, argmax=argmax)
    if stream is None:
        stream = _current_stream(C)
    elif not isinstance(stream, int):
        stream = stream.cuda_stream
    _check(_lib.spmm_run(plan, _addr(B), _addr(C), _addr(argmax), int(N), red, stream))


def spmm_plan_destroy(plan: int) -> None:
    _plan_dims.pop(plan, None)
    _check(_lib.spmm_plan_destroy(plan))


def spmm_plan_info(plan: int) -> dict:
    info = _Info()
    _check(_lib.spmm_plan_info(plan, ctypes.byref(info)))
    return {name: getattr(info, name) for name, _ in _Info._fields_}


def spmm_plan_route(plan: int, N: int, reduce) -> dict:
    red = REDUCE[reduce] if isinstance(reduce, str) else int(reduce)
    _check(_lib.spmm_plan_route(plan, int(N), red))
    return spmm_plan_info(plan)


def spmm_plan_partition(plan: int):
    """Row split as host numpy arrays: dict(n_heavy, seg_row, seg_begin, seg_end, light)."""
    import numpy as np
    counts = np.zeros(3, dtype=np.int64)
    z = ctypes.c_void_p(0)
    _check(_lib.spmm_plan_partition(plan, z, z, z, 0, z, 0, counts.ctypes.data))
    ns, nl = int(counts[1]), int(counts[2])
    sr = np.empty(ns, np.int64)
    sb = np.empty(ns, np.int64)
    se = np.empty(ns, np.int64)
    light = np.empty(nl, np.int64)
    _check(_lib.spmm_plan_partition(plan, sr.ctypes.data, sb.ctypes.data, se.ctypes.data, ns,
                                    light.ctypes.data, nl, counts.ctypes.data))
    return dict(n_heavy=int(counts[0]), seg_row=sr, seg_begin=sb, seg_end=se, light=light)


def spmm_plan_features(plan: int, V: int = 2) -> dict:
    """ParamSpMM Table 3 features of the plan's pattern (synchronous)."""
    f = _Features()
    _check(_lib.spmm_plan_features(plan, int(V), ctypes.byref(f)))
    return {name: getattr(f, name) for name, _ in _Features._fields_}


def spmm_set_mem_limit(nbytes: int) -> None:
    """Limit (bytes, 0 = none) on the device memory one library call of the
    calling thread may allocate."""
    _check(_lib.spmm_set_mem_limit(int(nbytes)))


def spmm_mem_stats() -> dict:
    m = _MemStats()
    _check(_lib.spmm_mem_stats(ctypes.byref(m)))
    return {name: getattr(m, name) for name, _ in _MemStats._fields_}


def spmm_plan_set_option(plan: int, option: int, value: int) -> None:
    _check(_lib.spmm_plan_set_option(plan, int(option), int(value)))


def spmm_coo_to_csr(row, col, val, M: int, K: int):
    """Stable edge-list -> CSR on the device: returns (rowptr, col, val) tensors."""
    import torch
    E = int(row.numel())
    _check_vector("row", row, "int64", exact_len=E)
    _check_vector("col", col, "int64", exact_len=E)
    _check_vector("val", val, "float32", exact_len=E)
    _check_gpu(row=row, col=col, val=val)
    dev = row.device
    rowptr = torch.empty(M + 1, dtype=torch.int64, device=dev)
    col_out = torch.empty(max(E, 1), dtype=torch.int64, device=dev)[:E]
    val_out = None if val is None else torch.empty(max(E, 1), dtype=torch.float32, device=dev)[:E]
    _check(_lib.spmm_coo_to_csr(_addr(row), _addr(col), _addr(val), E, int(M), int(K), _addr(rowptr),
                                _addr(col_out), _addr(val_out)))
    return rowptr, col_out, val_out


def spmm_coo_to_csr_noalloc(row, col, val, M: int, K: int, rowptr_out, col_out, val_out=None) -> None:
    """Edge-list -> CSR into the caller's tensors, with no device allocation
    in the library (at most 2^20 edges)."""
    E = int(row.numel())
    _check_vector("row", row, "int64", exact_len=E)
    _check_vector("col", col, "int64", exact_len=E)
    _check_vector("val", val, "float32", exact_len=E)
    _check_vector("rowptr_out", rowptr_out, "int64", exact_len=int(M) + 1)
    _check_vector("col_out", col_out, "int64", exact_len=E)
    _check_vector("val_out", val_out, "float32", exact_len=E if val is not None else None)
    if val is not None and val_out is None:
        raise ValueError("val_out is required with val")
    _check_gpu(row=row, col=col, val=val, rowptr_out=rowptr_out, col_out=col_out, val_out=val_out)
    _check(_lib.spmm_coo_to_csr_noalloc(_addr(row), _addr(col), _addr(val), E, int(M), int(K), _addr(rowptr_out),
                                        _addr(col_out), _addr(val_out)))


def spmm_plan_transpose(plan: int, scale: int = 0) -> int:
    h = _lib.spmm_plan_transpose(plan, int(scale))
    if not h:
        st, msg = spmm_last_error()
        raise SpmmError(st, msg)
    return h


def spmm_plan_reorder(plan: int, method: int = 1):
    """Reverse Cuthill-McKee permutation of a square plan as a device int64
    tensor: perm[i] = the node placed at position i (synchronous)."""
    import torch
    M = spmm_plan_info(plan)["M"]
    perm = torch.empty(M, dtype=torch.int64, device=torch.device("cuda", torch.cuda.current_device()))
    _check(_lib.spmm_plan_reorder(plan, int(method), _addr(perm) if M else None))
    return perm


def spmm_plan_permute(plan: int, perm) -> int:
    """Plan of P A P^T for a device int64 permutation (synchronous)."""
    M, _ = _dims(plan)
    _check_vector("perm", perm, "int64", exact_len=M)
    h = _lib.spmm_plan_permute(plan, _addr(perm) if perm is not None and perm.numel() else None)
    if not h:
        st, msg = spmm_last_error()
        raise SpmmError(st, msg)
    return h


def spmm_max_backward(plan_t: int, argmax, dC, dB, N: int, stream=None) -> None:
    """dB [K, N] of a max aggregation; plan_t is the transpose [K, M] of the
    forward adjacency, argmax and dC are [M, N]."""
    _check_matrix("argmax", argmax, "int64", None, int(N))
    _check_matrix("dC", dC, "float32", None, int(N))
    _check_matrix("dB", dB, "float32", None, int(N))
    Mt, Kt = _dims(plan_t)
    _check_rows("argmax", argmax, Kt)
    _check_rows("dC", dC, Kt)
    _check_rows("dB", dB, Mt)
    _check_gpu(argmax=argmax, dC=dC, dB=dB)
    if stream is None:
        stream = _current_stream(dB)
    elif not isinstance(stream, int):
        stream = stream.cuda_stream
    _check(_lib.spmm_max_backward(plan_t, _addr(argmax), _addr(dC), _addr(dB), int(N), stream))


class SparseAdj:
    """A CSR adjacency held once on the GPU and applied many times
    (graph-spmm card, "Usage": build the CSR once, apply it per layer)."""

    def __init__(self, rowptr, col, val=None, num_cols: Optional[int] = None, _plan: Optional[int] = None):
        if _plan is not None:                      # wraps an existing plan (a transpose)
            self._plan = _plan
            info = spmm_plan_info(_plan)
            self.M, self.K = int(info["M"]), int(info["K"])
            self.weighted = bool(info["has_val"])
            self.device = None
        else:
            self.M = int(rowptr.numel()) - 1
            self.K = int(num_cols if num_cols is not None else self.M)
            self.device = rowptr.device
            self.weighted = val is not None
            self._plan = spmm_plan_create(rowptr, col, val, self.M, self.K)
        self._transposes = {}

    @classmethod
    def from_edge_index(cls, edge_index, num_nodes: int, val=None, num_cols: Optional[int] = None):
        """CSR from a [2, E] edge list: entry (edge_index[0][e], edge_index[1][e])
        keeps its edge-list position within its row (graph-spmm card, API table)."""
        K = int(num_cols if num_cols is not None else num_nodes)
        row = edge_index[0].contiguous()
        col = edge_index[1].contiguous()
        rowptr, c, v = spmm_coo_to_csr(row, col, None if val is None else val.contiguous(), int(num_nodes), K)
        return cls(rowptr, c, v, num_cols=K)

    def transpose(self, scale_by_inverse_degree: bool = False) -> "SparseAdj":
        """A^T as its own plan (cached); scaled by 1/deg for the mean's backward."""
        key = int(bool(scale_by_inverse_degree))
        if key not in self._transposes:
            self._transposes[key] = SparseAdj(None, None, _plan=spmm_plan_transpose(self._plan, key))
        return self._transposes[key]

    @property
    def plan(self) -> int:
        return self._plan

    def info(self) -> dict:
        return spmm_plan_info(self._plan)

    def set_option(self, option: int, value: int) -> None:
        spmm_plan_set_option(self._plan, option, value)

    def features(self, V: int = 2) -> dict:
        """ParamSpMM Table 3 features of the adjacency (synchronous)."""
        return spmm_plan_features(self._plan, V)

    def reordered(self):
        """(P A P^T as a new SparseAdj, perm) with the reverse Cuthill-McKee order:
        perm[i] = the node placed at position i; use B[perm] as its features and
        C_new[inv] (inv[perm] = arange) to return to the original numbering."""
        perm = spmm_plan_reorder(self._plan)
        return SparseAdj(None, None, _plan=spmm_plan_permute(self._plan, perm)), perm

    def reduce(self, B, reduce: str = "sum", out=None, argmax=None, stream=None):
        import torch
        if B.dim() != 2 or B.shape[0] != self.K:
            raise ValueError(f"B has shape {tuple(B.shape)}, expected ({self.K}, N)")
        N = int(B.shape[1])
        if out is not None and tuple(out.shape) != (self.M, N):
            raise ValueError(f"out has shape {tuple(out.shape)}, expected ({self.M}, {N})")
        if out is None:
            out = torch.empty((self.M, N), dtype=torch.float32, device=B.device)
        if reduce == "max" and argmax is None:
            argmax = torch.empty((self.M, N), dtype=torch.int64, device=B.device)
        spmm_run(self._plan, B, out, argmax if reduce == "max" else None, N, reduce, stream)
        return (out, argmax) if reduce == "max" else out

    def __matmul__(self, B):
        return self.reduce(B, "sum")

    def max_backward(self, argmax, dC, out=None, stream=None):
        """dB for a max aggregation over this (unweighted) adjacency."""
        import torch
        N = int(dC.shape[1])
        _check_matrix("dC", dC, "float32", self.M, N)
        _check_matrix("argmax", argmax, "int64", self.M, N)
        _check_matrix("out", out, "float32", self.K, N)
        _check_gpu(dC=dC, argmax=argmax, out=out)
        if out is None:
            out = torch.empty((self.K, N), dtype=torch.float32, device=dC.device)
        spmm_max_backward(self.transpose().plan, argmax, dC, out, N, stream)
        return out

    def close(self) -> None:
        for t in self._transposes.values():
            t.close()
        self._transposes = {}
        if self._plan:
            spmm_plan_destroy(self._plan)
            self._plan = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def aggregate(adj: SparseAdj, B, reduce: str = "sum"):
    """Differentiable aggregation: forward and backward both run in the HIP
    library (backward of sum / mean: the transposed product, of max: the
    argmax scatter).  Returns C (and, for max, the argmax as a second output
    without a gradient)."""
    import torch

    class _Aggregate(torch.autograd.Function):
        @staticmethod
        def forward(ctx, B_):
            out = adj.reduce(B_.contiguous(), reduce)
            if reduce == "max":
                C, arg = out
                ctx.save_for_backward(arg)
                ctx.mark_non_differentiable(arg)
                return C, arg
            return out

        @staticmethod
        def backward(ctx, dC, *unused):
            dC = dC.contiguous()
            if reduce == "max":
                (arg,) = ctx.saved_tensors
                return adj.max_backward(arg, dC)
            return adj.transpose(scale_by_inverse_degree=(reduce == "mean")).reduce(dC, "sum")

    return _Aggregate.apply(B)

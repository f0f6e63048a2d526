"""C ABI of the HIP library, without a GPU: it loads, exports every function the
header declares, and rejects bad arguments before touching the device."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spmm.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spmm_[a-z_]+)\s*\(", text)))


def test_header_declares_the_documented_calls():
    names = _declared_functions()
    for required in ("spmm_plan_create", "spmm_run", "spmm_plan_destroy", "spmm_plan_info",
                     "spmm_plan_route", "spmm_plan_partition", "spmm_plan_set_option",
                     "spmm_last_error"):
        assert required in names


def test_library_exports_every_declared_symbol():
    import gnn_sparse_dense_amd as G
    lib = G.lib()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert sorted(G.EXPORTED) == _declared_functions()
    out = subprocess.run(["nm", "-D", "--defined-only", G.LIB_PATH], capture_output=True, text=True).stdout
    exported = sorted(set(re.findall(r" T (spmm_\w+)", out)))
    assert exported == _declared_functions(), "exported C symbols differ from the header"


def test_header_compiles_as_c():
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-x", "c", HEADER],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


@pytest.mark.parametrize("struct,cls", [("spmm_plan_info", "_Info"), ("spmm_features", "_Features"),
                                        ("spmm_mem_stats", "_MemStats")])
def test_header_struct_layout_matches_binding(struct, cls, tmp_path):
    import gnn_sparse_dense_amd as G
    py = getattr(G, cls)
    fields = [name for name, _ in py._fields_]
    body = "".join(f'printf("%zu\\n", offsetof(struct {struct}, {f}));' for f in fields)
    src = ('#include <stdio.h>\n#include <stddef.h>\n#include "spmm.h"\n'
           f'int main(void){{printf("%zu\\n", sizeof(struct {struct}));{body}return 0;}}\n')
    c = tmp_path / "layout_probe.c"
    exe = tmp_path / "layout_probe"
    c.write_text(src)
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(c), "-o", str(exe)], check=True)
    vals = list(map(int, subprocess.run([str(exe)], capture_output=True, text=True).stdout.split()))
    assert vals[0] == ctypes.sizeof(py), (struct, vals[0], ctypes.sizeof(py))
    for f, off in zip(fields, vals[1:]):
        assert off == getattr(py, f).offset, (struct, f)


def _err():
    import gnn_sparse_dense_amd as G
    return G.spmm_last_error()


def test_argument_errors_without_gpu():
    import gnn_sparse_dense_amd as G
    lib = G.lib()
    # plan creation: negative sizes and a NULL row pointer fail before any HIP call
    assert lib.spmm_plan_create(None, None, None, -1, 5) is None
    assert _err()[0] == G.SPMM_E_INVALID_ARG
    assert lib.spmm_plan_create(None, None, None, 4, 4) is None
    st, msg = _err()
    assert st == G.SPMM_E_INVALID_ARG and "rowptr" in msg
    assert lib.spmm_plan_create(None, None, None, 2**31, 4) is None
    assert _err()[0] == G.SPMM_E_UNSUPPORTED
    # runs on a NULL plan, bad N, bad reduce
    assert lib.spmm_run(None, None, None, None, 8, 0, None) == G.SPMM_E_INVALID_ARG
    fake = ctypes.c_void_p(0x1000)      # never dereferenced: checks come first
    assert lib.spmm_run(fake, None, None, None, 0, 0, None) == G.SPMM_E_INVALID_ARG
    assert "N must be positive" in _err()[1]
    assert lib.spmm_run(fake, None, None, None, 8, 7, None) == G.SPMM_E_INVALID_ARG
    assert lib.spmm_run(fake, None, None, fake, 8, G.SPMM_SUM, None) == G.SPMM_E_INVALID_ARG
    assert "argmax" in _err()[1]
    assert lib.spmm_plan_info(None, None) == G.SPMM_E_INVALID_ARG
    assert lib.spmm_plan_set_option(None, 1, 5) == G.SPMM_E_INVALID_ARG
    assert lib.spmm_plan_route(None, 8, 0) == G.SPMM_E_INVALID_ARG
    assert lib.spmm_plan_partition(None, None, None, None, 0, None, 0, None) == G.SPMM_E_INVALID_ARG
    assert lib.spmm_plan_destroy(None) == G.SPMM_OK
    assert _err()[0] == G.SPMM_OK


def test_binding_rejects_strided_or_mistyped_tensors():
    """The C ABI sees only pointers, so the binding refuses tensors whose
    memory is not the packed row-major matrix the library reads or writes
    (checked before any HIP call)."""
    import torch

    import gnn_sparse_dense_amd as G
    C = torch.zeros((4, 8), dtype=torch.float32)
    strided = torch.zeros((8, 6), dtype=torch.float32).t()          # [6, 8], column-major
    with pytest.raises(ValueError, match="contiguous"):
        G.spmm_run(0, strided, C, None, 8, "sum")
    with pytest.raises(TypeError, match="float32"):
        G.spmm_run(0, torch.zeros((6, 8), dtype=torch.float64), C, None, 8, "sum")
    with pytest.raises(ValueError, match="shape"):
        G.spmm_run(0, torch.zeros((6, 7), dtype=torch.float32), C, None, 8, "sum")
    with pytest.raises(TypeError, match="int64"):
        G.spmm_run(0, torch.zeros((6, 8)), C, torch.zeros((4, 8), dtype=torch.int32), 8, "max")
    with pytest.raises(ValueError, match="shape"):
        G.spmm_run(0, torch.zeros((6, 8)), C, torch.zeros((5, 8), dtype=torch.int64), 8, "max")
    G._plan_dims[0x1000] = (4, 6)          # a handle the library never sees
    try:
        with pytest.raises(ValueError, match="GPU"):
            G.spmm_run(0x1000, torch.zeros((6, 8)), C, None, 8, "sum")
    finally:
        G._plan_dims.pop(0x1000)


def test_binding_rejects_wrong_row_counts():
    """Row counts of B, C, argmax, dC and dB, and the lengths of the CSR and
    edge-list arrays, are checked on the host before any address reaches the
    library (an undersized tensor would otherwise be read or written out of
    bounds)."""
    import torch

    import gnn_sparse_dense_amd as G
    fake = 0x2000                              # never dereferenced: checks come first
    G._plan_dims[fake] = (4, 6)                # plan of A [4, 6]
    try:
        B = torch.zeros((6, 8))
        C = torch.zeros((4, 8))
        with pytest.raises(ValueError, match="B has 5 rows, expected 6"):
            G.spmm_run(fake, torch.zeros((5, 8)), C, None, 8, "sum")
        with pytest.raises(ValueError, match="C has 3 rows, expected 4"):
            G.spmm_run(fake, B, torch.zeros((3, 8)), None, 8, "sum")
        with pytest.raises(ValueError, match="argmax has"):
            G.spmm_run(fake, B, C, torch.zeros((3, 8), dtype=torch.int64), 8, "max")
        # max backward over the transpose plan [6, 4]: argmax / dC [4, N], dB [6, N]
        G._plan_dims[fake] = (6, 4)
        arg = torch.zeros((4, 8), dtype=torch.int64)
        with pytest.raises(ValueError, match="dC has 5 rows, expected 4"):
            G.spmm_max_backward(fake, arg, torch.zeros((5, 8)), torch.zeros((6, 8)), 8)
        with pytest.raises(ValueError, match="argmax has 3 rows, expected 4"):
            G.spmm_max_backward(fake, arg[:3], torch.zeros((4, 8)), torch.zeros((6, 8)), 8)
        with pytest.raises(ValueError, match="dB has 5 rows, expected 6"):
            G.spmm_max_backward(fake, arg, torch.zeros((4, 8)), torch.zeros((5, 8)), 8)
        G._plan_dims[fake] = (6, 6)
        with pytest.raises(ValueError, match="perm has 5 elements, expected 6"):
            G.spmm_plan_permute(fake, torch.zeros(5, dtype=torch.int64))
    finally:
        G._plan_dims.pop(fake)
    # CSR arrays: rowptr must hold M + 1 entries, col and val at least rowptr[M]
    rowptr = torch.tensor([0, 2, 3], dtype=torch.int64)
    with pytest.raises(ValueError, match="rowptr has 3 elements, expected 4"):
        G.spmm_plan_create(rowptr, torch.zeros(3, dtype=torch.int64), None, 3, 3)
    with pytest.raises(ValueError, match="col has 2 elements, fewer than the 3"):
        G.spmm_plan_create(rowptr, torch.zeros(2, dtype=torch.int64), None, 2, 3)
    with pytest.raises(ValueError, match="val has 1 elements, fewer than the 3"):
        G.spmm_plan_create(rowptr, torch.zeros(3, dtype=torch.int64), torch.zeros(1), 2, 3)
    # edge lists: row, col and val of one length
    with pytest.raises(ValueError, match="col has 3 elements, expected 4"):
        G.spmm_coo_to_csr(torch.zeros(4, dtype=torch.int64), torch.zeros(3, dtype=torch.int64), None, 2, 2)
    with pytest.raises(ValueError, match="val has 2 elements, expected 4"):
        G.spmm_coo_to_csr(torch.zeros(4, dtype=torch.int64), torch.zeros(4, dtype=torch.int64), torch.zeros(2),
                          2, 2)


def test_last_error_truncates():
    import gnn_sparse_dense_amd as G
    lib = G.lib()
    lib.spmm_run(None, None, None, None, 8, 0, None)
    buf = ctypes.create_string_buffer(6)
    assert lib.spmm_last_error(buf, 6) == G.SPMM_E_INVALID_ARG
    assert len(buf.value) == 5


def test_product_path_does_not_touch_the_oracle():
    """The HIP package and its sources never import or link the oracle."""
    pkg = os.path.join(ROOT, "gnn_sparse_dense_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower(), f"{f} mentions the oracle"

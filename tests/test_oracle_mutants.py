"""Plant plausible mistakes in copies of the oracle and require the pins to notice.

Each mutant is a one-line textual change to oracle/spmm_oracle.c (a dropped
term, a wrong sign, a transposed operand, a wrong tie rule, an off-by-one in
the row split, ...), compiled with gcc into a temporary library.  The test
passes only if at least one pin in tests/oracle_pins.py fails on it, which is
evidence that the pins constrain every part of the oracle.
"""
import os

import pytest

import oracle
from oracle import build as obuild
from tests.oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "spmm_oracle.c")

MUTANTS = {
    "dropped_last_term": ("for (int64_t p = first; p < last; ++p) {\n                    float b",
                          "for (int64_t p = first; p < last - 1; ++p) {\n                    float b"),
    "wrong_sign": ("acc = acc + product(val, p, b);", "acc = acc - product(val, p, b);"),
    "transposed_B": ("float b = B[col[p] * N + k];", "float b = B[k * K + col[p]];"),
    "weight_ignored": ("return val[p] * b;", "return b;"),
    "later_tie_wins": ("if (t > best) {", "if (t >= best) {"),
    "argmax_is_position": ("arg = col[p];", "arg = p;"),
    "empty_max_arg_zero": ("int64_t arg = -1;", "int64_t arg = 0;"),
    "mean_divisor_off": ("acc / (float)deg", "acc / (float)(deg + 1)"),
    "max_skips_first": ("float best = product(val, first, B[col[first] * N + k]);",
                        "float best = -1e30f;"),
    "heavy_threshold_ge": ("if (deg > T) {", "if (deg >= T) {"),
    "piece_overlap": ("int64_t e = b + L;", "int64_t e = b + L + 1;"),
    "sample_variance": ("var = (M > 0) ? var / (double)M : 0.0;",
                        "var = (M > 1) ? var / (double)(M - 1) : 0.0;"),
    "gap_as_printed": ("if (tr == 0) return 0;", ""),
    "validate_skips_last_row": ("for (int64_t i = 0; i < M; ++i)\n        for (int64_t p = rowptr[i]; p < rowptr[i + 1]; ++p)\n            if (col[p] < 0",
                                "for (int64_t i = 0; i + 1 < M; ++i)\n        for (int64_t p = rowptr[i]; p < rowptr[i + 1]; ++p)\n            if (col[p] < 0"),
    "sumabs_signed": ("s += fabs(a * (double)B[col[p] * N + k]);", "s += a * (double)B[col[p] * N + k];"),
    "coo_unstable": ("int64_t p = cursor[row[e]]++;", "int64_t p = rowptr_out[row[e] + 1] - 1 - (cursor[row[e]]++ - rowptr_out[row[e]]);"),
    "transpose_scale_off": ("val_t[q] = scale ? a / (float)deg : a;", "val_t[q] = scale ? a / (float)(deg + 1) : a;"),
    "max_backward_skips_row0": ("for (int64_t i = 0; i < M; ++i)\n        for (int64_t k = 0; k < N; ++k) {\n            int64_t j",
                                "for (int64_t i = 1; i < M; ++i)\n        for (int64_t k = 0; k < N; ++k) {\n            int64_t j"),
    "features_bandwidth_stored_order": ("                if (col[p] < lo) lo = col[p];\n", ""),
    "features_cv_all_rows": ("if (d > 0) var_ne += (d - mean_ne) * (d - mean_ne);",
                             "var_ne += (d - mean_ne) * (d - mean_ne);"),
    "features_padding_counts_duplicates": ("1.0 - (double)distinct / ((double)vectors * (double)V)",
                                           "1.0 - (double)nnz / ((double)vectors * (double)V)"),
    "features_block_skips_first_row": ("for (int64_t i = g * V; i < g * V + V && i < M; ++i)",
                                       "for (int64_t i = g * V + 1; i < g * V + V && i < M; ++i)"),
    "rcm_not_reversed": ("for (int64_t i = 0; i < M; ++i) perm[i] = queue[M - 1 - i];",
                         "for (int64_t i = 0; i < M; ++i) perm[i] = queue[i];"),
    "rcm_children_unsorted": ("            qsort(queue + first, (size_t)(tail - first), sizeof(int64_t), cmp_deg_id);\n", ""),
    "rcm_largest_degree_first": ("if (g_deg[x] != g_deg[y]) return (g_deg[x] > g_deg[y]) - (g_deg[x] < g_deg[y]);",
                                 "if (g_deg[x] != g_deg[y]) return (g_deg[x] < g_deg[y]) - (g_deg[x] > g_deg[y]);"),
    "rcm_degree_counts_duplicates": ("        deg[i] = w - b;", "        deg[i] = n;"),
    "permute_columns_not_renamed": ("buf[q].c = inv[col[rowptr[o] + q]];", "buf[q].c = col[rowptr[o] + q];"),
    "fused_is_unfused": ("acc = fmaf(val[p], b, acc);", "acc = acc + val[p] * b;"),
    "unfused_is_fused": ("acc = acc + product(val, p, b);", "acc = fmaf(val ? val[p] : 1.0f, b, acc);"),
    "permute_rows_unsorted": ("        qsort(buf, (size_t)n, sizeof(cp_pair), cmp_cp);\n", ""),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    before, after = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(before) == 1, f"mutation site for {name} not unique"
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(before, after))
    lib = obuild.build(str(src), str(tmp_path / "libmutant.so"))
    orc = oracle.Oracle(lib)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"

// Host-side plan of the CSR SpMM library: the device buffers a plan owns, its
// descriptors, options and last routing decision.  Only the C ABI
// implementation (api.cpp) uses it; kernels see their argument structs.
#pragma once

#include "spmm_internal.h"

namespace gspmm {

struct Route {
    int lanes = 64, vec = 4, coarsen = 1, slices = 1;
    int xcd_remap = 1, nt_store = 0;
    bool split = false;
    bool tiled = false;
    bool compact = false;
    bool window = false;
    bool window_sorted = false;   // the window kernel for rows in column order
    bool mfma = false;
    bool pairs = false;
    bool merge = false;
    bool fused_split = false;     // light rows and pieces went out in one dispatch
};

// V = 2 panels are used by default only up to this padding share of vector
// slots (1 - nnz / (2 * vectors)).
constexpr double kPairMaxPadding = 0.3;

}  // namespace gspmm

struct spmm_plan {
    int device = 0;
    int num_cus = 256;            // compute units of the plan's device
    int64_t M = 0, K = 0, nnz = 0;
    // descriptors
    int64_t dmax = 0, n_empty = 0, sum_deg2 = 0;
    double mean_deg = 0, cv_deg = 0, plan_ms = 0;
    // narrowed CSR (device)
    int *rowptr = nullptr;
    int *col = nullptr;
    float *val = nullptr;
    // row split (device)
    bool split = false;
    int64_t T = 0, L = 0, n_heavy = 0, n_seg = 0, n_light = 0;
    int *heavy_rows = nullptr, *seg_first = nullptr, *seg_begin = nullptr, *seg_end = nullptr;
    int *seg_order = nullptr;     // pieces in the order they run (column of their first entry)
    float *partial = nullptr;
    int *part_arg = nullptr;
    // row-tile records (low-degree graphs)
    int *tiles = nullptr;
    int tile_cap = 0, tile_words = 0;
    bool tile_compact = false;
    int64_t tile_overflow = 0;
    double win_frac = 0;       // share of entries inside their row's kWinRows block
    bool rows_sorted = false;  // every row's columns are non-decreasing
    int *win_lo = nullptr, *win_in = nullptr;   // per-row run lengths (sorted rows)
    // fp16 community tiles + residual CSR (built on request)
    uint4 *mfma_tiles = nullptr;
    uint4 *mfma_tiles_lo = nullptr;   // split tiles only
    int *mfma_tile_exp = nullptr;     // split tiles only
    int *mfma_rowptr = nullptr, *mfma_col = nullptr;
    float *mfma_val = nullptr;
    int64_t mfma_rnnz = 0;
    // V = 2 panels (built on request)
    int *pair_prow = nullptr;
    unsigned *pair_col = nullptr;
    float *pair_val = nullptr;
    int64_t pair_nvec = 0;
    bool pair_unsorted = false;
    // merge-path segments (built on request)
    int *merge_seg_row = nullptr, *merge_seg_entry = nullptr, *merge_carry_row = nullptr, *merge_carry_arg = nullptr;
    float *merge_carry = nullptr;
    int64_t merge_nseg = 0;
    // options (-1 / 0 = automatic)
    int64_t opt_T = -1, opt_L = -1, opt_split = -1, opt_tiles = -1, opt_window = -1;
    int opt_lanes = 0, opt_coarsen = 0, opt_vec = 0, opt_xcd = -1, opt_nt = -1, opt_mfma = 0, opt_vblock = -1, opt_balance = 0, opt_piece_order = 1, opt_split_fused = 1;
    // device memory limit of calls on this plan (<= 0: none), and the count
    // of changes to the set of its device buffers
    int64_t mem_limit = 0;
    int64_t generation = 0;
    // last routing decision
    int64_t route_N = 0;
    gspmm::Route route;
};

// Host-side declarations shared by the translation units of the gfx950 CSR
// SpMM library: the kernel lookup table and the launchers of the plan-time,
// graph-construction, feature and product kernels (kernel constants and
// argument structs are in kernels.h, the plan in plan.h).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "kernels.h"
#include "merge_args.h"
#include "mfma_args.h"
#include "pair_args.h"
#include "spmm.h"

namespace gspmm {

// Looks up a compiled row kernel; nullptr when the combination is not built.
RowKernelFn row_kernel_v1(const RowKernelKey &k);
RowKernelFn row_kernel_v2(const RowKernelKey &k);
RowKernelFn row_kernel_v4(const RowKernelKey &k);
RowKernelFn row_kernel(const RowKernelKey &k);

hipError_t launch_combine(const CombineArgs &a, bool is_max, hipStream_t s);
// Pieces and light rows of a split product in one dispatch (split_fused.hip);
// available for the light-row shapes below.  *launched is false (and nothing
// runs) when the shapes or the grid do not fit one launch: launch separately.
bool split_fused_available(int lanes, int vec, int coarsen);
hipError_t launch_split_fused(int lanes, bool has_val, bool is_max, const RowArgs &light, const RowArgs &pieces,
                              int light_slices, hipStream_t s, bool *launched);
hipError_t launch_window(const RowArgs &a, bool has_val, bool is_max, bool sorted, hipStream_t s);

// ---- plan-time kernels (plan_kernels.hip) ----
struct RowScanOut {        // one record per scan block
    int64_t bad_row;       // first row breaking monotonicity, or INT64_MAX
    int64_t sum_deg;
    int64_t sum_deg2;
    int64_t dmax;
    int64_t n_empty;
};
hipError_t launch_rowscan(const int64_t *rowptr, int64_t M, int *rowptr32, RowScanOut *out,
                          int64_t nblocks, hipStream_t s);
hipError_t launch_colscan(const int64_t *col, int64_t nnz, int64_t K, int *col32,
                          int64_t *bad_pos, int64_t nblocks, hipStream_t s);

struct PartCount {         // one record per scan block
    int64_t n_heavy, n_seg, n_light;
};
hipError_t launch_part_count(const int *rowptr32, int64_t M, int64_t T, int64_t L,
                             PartCount *out, int64_t nblocks, hipStream_t s);
hipError_t launch_part_write(const int *rowptr32, int64_t M, int64_t T, int64_t L,
                             const PartCount *offsets, int *heavy_rows, int *seg_first,
                             int *seg_begin, int *seg_end, int *light_rows, int64_t nblocks,
                             hipStream_t s);

// Order in which the pieces run: ascending column of each piece's first
// entry, ties by piece id (synchronous; allocates its own sort buffers).
hipError_t build_piece_order(const int *col, const int *seg_begin, int64_t n_seg, int *order);

hipError_t launch_window_runs(const int *rowptr, const int *col, int64_t M, int *win_lo, int *win_in,
                              hipStream_t s);
hipError_t launch_window_scan(const int *rowptr, const int *col, int64_t M, int64_t *out, int64_t nblocks,
                              hipStream_t s);
hipError_t launch_tile_build(const int *rowptr, const int *col, const float *val, int64_t M, int cap, int rs,
                             bool compact, int *tiles, int64_t *overflow, int64_t nblocks, hipStream_t s);
int64_t tile_build_blocks(int64_t M);

// ---- fp16 matrix-core tiles for community blocks (mfma_tile.hip) ----
hipError_t mfma_build_tiles(const int *rowptr, const int *col, const float *val, int64_t M, uint4 *atiles,
                            uint4 *atiles_lo, int *tile_exp, int64_t ntiles, int *rrowptr, int *range_flag,
                            hipStream_t s);
hipError_t mfma_write_residual(const int *rowptr, const int *col, const float *val, int64_t M,
                               const int *rrowptr, int *rcol, float *rval, hipStream_t s);
hipError_t launch_mfma(const MfmaArgs &a, bool has_val, hipStream_t s);

// ---- V = 2 vectorized blocking (pair_kernel.hip) ----
struct PairOutput {
    unsigned *pcol;   // device, allocated by pair_build
    float *pval;      // device, allocated when weighted
    int nvec;         // nonzero vectors
    int unsorted;     // some row is not stored with ascending columns
};
// rows_sorted: every row is stored with ascending columns (merge build, no sort).
hipError_t pair_build(const int *rowptr, const int *col, const float *val, int64_t M, int64_t K, int64_t nnz,
                      bool rows_sorted, int *prow, PairOutput *out);
// Nonzero vectors of the V = 2 panels when every row is stored with ascending
// columns (a merge per panel, no sort; synchronous).
hipError_t pair_count_sorted(const int *rowptr, const int *col, int64_t M, int64_t *vectors);
PairKernelFn pair_kernel(int lanes, int vec, bool has_val, bool is_max);
hipError_t launch_pairs(PairKernelFn fn, PairArgs a, int lanes, int slices, hipStream_t s);

// ---- merge-path balancing (merge_kernel.hip) ----
hipError_t merge_build(const int *rowptr, int64_t M, int64_t nnz, int64_t nseg, int *seg_row, int *seg_entry);
MergeKernelFn merge_kernel(int vec, bool has_val, bool is_max);
hipError_t launch_merge(MergeKernelFn fn, const MergeArgs &a, int vec, bool is_max, hipStream_t s);

// ---- locality reordering (reorder.hip) ----
hipError_t rcm_order(const int *rowptr, const int *col, int64_t M, int64_t nnz, int64_t *perm, int64_t *levels);
hipError_t permute_csr(const int *rowptr, const int *col, const float *val, int64_t M, int64_t nnz,
                       const int64_t *perm, int64_t *rowptr_p, int64_t *col_p, float *val_p, bool *bad_perm);

// ---- pattern features (features.hip) ----
struct FeatureRecord {   // one per block, folded on the host in block order
    int64_t a, b, c;
};
hipError_t pattern_features(const int *rowptr, const int *col, int64_t M, int64_t K, int64_t nnz, int64_t V,
                            int64_t *bw_sum, int64_t *bw_max, int64_t *nonempty, int64_t *distinct,
                            int64_t *vectors);

// ---- graph construction and backward (transform.hip) ----
struct MaxGradArgs {
    const int *rowptr_t;     // int32 [rows+1]: transposed (unweighted) CSR
    const int *col_t;        // int32 [nnz]: source rows i, ascending within a row
    const int64_t *argmax;   // int64 [M, N] from the forward max
    const float *dC;         // fp32 [M, N]
    float *dB;               // fp32 [rows, N]
    int64_t rows;            // rows of the transpose (= columns K of the forward)
    int64_t N;
};
// Device and host workspace of an edge-list sort (coo_check_blocks(E)
// records for the range check, hipCUB storage of coo_sort_storage_bytes).
struct CooWorkspace {
    int *keys = nullptr, *idx = nullptr, *skeys = nullptr, *perm = nullptr;   // int32 [E] each
    int64_t *bad = nullptr;          // device [coo_check_blocks(E)]
    int64_t *bad_host = nullptr;     // host [coo_check_blocks(E)]
    void *sort = nullptr;
    size_t sort_bytes = 0;
};
int64_t coo_check_blocks(int64_t E);
hipError_t coo_sort_storage_bytes(int64_t E, int64_t M, size_t *bytes);
hipError_t coo_to_csr_in(const int64_t *row, const int64_t *col, const float *val, int64_t E, int64_t M, int64_t K,
                         int64_t *rowptr_out, int64_t *col_out, float *val_out, int64_t *first_bad,
                         const CooWorkspace &w, hipStream_t s);
// The allocation-free variant: workspace in a fixed device array of
// kNoAllocScratchBytes per device, edge lists of at most kNoAllocMaxEdges;
// *too_large = 1 (and nothing launched) beyond that.
constexpr int64_t kNoAllocMaxEdges = int64_t(1) << 20;
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
hipError_t coo_to_csr_noalloc(const int64_t *row, const int64_t *col, const float *val, int64_t E, int64_t M,
                              int64_t K, int64_t *rowptr_out, int64_t *col_out, float *val_out, int64_t *first_bad,
                              int *too_large);
hipError_t coo_to_csr(const int64_t *row, const int64_t *col, const float *val, int64_t E, int64_t M, int64_t K,
                      int64_t *rowptr_out, int64_t *col_out, float *val_out, int64_t *first_bad, hipStream_t s);
hipError_t transpose_csr(const int *rowptr, const int *col, const float *val, int64_t M, int64_t K, int64_t nnz,
                         bool scale, int64_t *rowptr_t, int64_t *col_t, float *val_t, hipStream_t s);
hipError_t launch_maxgrad(const MaxGradArgs &a, hipStream_t s);

}  // namespace gspmm

// Internal declarations of the gfx950 CSR SpMM library: plan layout, kernel
// arguments and the launch table shared by the HIP translation units.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "spmm.h"

namespace gspmm {

constexpr int kBlock = 256;             // threads per block: 4 wave64s
constexpr int kWaves = kBlock / 64;
constexpr int kChunk = 256;             // col/val entries a wave stages in LDS at once
constexpr int kPartialWidth = 256;      // columns per pass of the split path
constexpr int kRowsPerScanBlock = 1024; // rows per block of the plan-time scans
constexpr int kXcds = 8;                // MI355X: 8 XCDs, 32 CUs each
constexpr int kXcdChunk = 64;           // consecutive blocks one XCD takes at a time
constexpr int kTileRows = 8;            // rows per row-tile record
constexpr int kTileLdsWords = 512;      // LDS words per wave for row-tile records (2 records)
constexpr int kTileMaxCap = 120;        // largest entries per row-tile record
constexpr int kWinRows = 256;           // rows of a community window
constexpr int kWinCols = 64;            // B columns staged per window block
constexpr int kWinBlock = 1024;         // threads of a window block
constexpr int kWinChunk = 128;          // staged entries per wave in window blocks
constexpr int kMfmaKSteps = kWinRows / 16;   // k-steps of 16 per 256-wide community tile
constexpr int kMfmaBtPitch = kWinRows + 8;   // fp16 per staged B^T row (16-byte skew per row)

// Arguments of the row kernel (light rows or split pieces).
struct RowArgs {
    const int *rowptr;     // int32 [M+1]                     (row mode)
    const int *seg_begin;  // int32 [n_seg]                    (piece mode)
    const int *seg_end;    // int32 [n_seg]                    (piece mode)
    const int *col;        // int32 [nnz]
    const float *val;      // fp32 [nnz] or nullptr
    const int *tiles;      // row-tile records (tile kernels only)
    int tile_cap;          // entries per record
    int tile_words;        // record length in int32 words
    const float *B;        // fp32 [K, N]
    float *out;            // C (row mode) or the partial buffer (piece mode)
    int64_t *argmax;       // int64 [M, N] or nullptr          (row mode, max)
    int *part_arg;         // int32 partial argmax             (piece mode, max)
    int64_t ldo;           // row stride of out / argmax / part_arg, in elements
    int64_t N;             // columns of B (row stride of B)
    int64_t K;             // rows of B
    int64_t c_begin;       // first column handled by this launch
    int64_t c_end;         // one past the last column handled
    int64_t task_base;     // first task of this launch
    int64_t ntasks;        // rows (row mode) or pieces (piece mode): tasks end here
    int skip_above;        // row mode: rows longer than this are split, not written here
    int mean;              // divide by the row degree (row mode)
    int xcd_remap;         // give each XCD a contiguous range of tasks
    int nt_store;          // non-temporal output stores
};

// Arguments of the ordered combine of split pieces.
struct CombineArgs {
    const int *heavy_rows;   // int32 [n_heavy]
    const int *seg_first;    // int32 [n_heavy+1]: pieces of heavy row h
    const int *rowptr;       // int32 [M+1]
    const float *partial;    // fp32 [n_seg, kPartialWidth]
    const int *part_arg;     // int32 [n_seg, kPartialWidth] (max only)
    float *C;                // fp32 [M, N]
    int64_t *argmax;         // int64 [M, N] or nullptr
    int64_t N;
    int64_t c_begin, c_end;  // columns of this pass (c_end - c_begin <= kPartialWidth)
    int64_t n_heavy;
    int mean;
};

struct RowKernelKey {
    int lanes;    // G: lanes per row (4..64); 64 / G rows per wave
    int vec;      // floats per lane access (1, 2, 4)
    int coarsen;  // F: accesses per lane per entry
    bool has_val;
    bool is_max;
    bool pieces;  // piece mode (split rows) instead of row mode
    bool tiled;   // row-tile records instead of CSR row bounds
    bool compact; // compact (16-bit) row-tile records
};

typedef void (*RowKernelFn)(RowArgs);

// Looks up a compiled row kernel; nullptr when the combination is not built.
RowKernelFn row_kernel_v1(const RowKernelKey &k);
RowKernelFn row_kernel_v2(const RowKernelKey &k);
RowKernelFn row_kernel_v4(const RowKernelKey &k);
RowKernelFn row_kernel(const RowKernelKey &k);

hipError_t launch_combine(const CombineArgs &a, bool is_max, hipStream_t s);
hipError_t launch_window(const RowArgs &a, bool has_val, bool is_max, hipStream_t s);

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

hipError_t launch_window_scan(const int *rowptr, const int *col, int64_t M, int64_t *out, int64_t nblocks,
                              hipStream_t s);
hipError_t launch_tile_build(const int *rowptr, const int *col, const float *val, int64_t M, int cap, int rs,
                             bool compact, int *tiles, int64_t *overflow, int64_t nblocks, hipStream_t s);
int64_t tile_build_blocks(int64_t M);

// ---- fp16 matrix-core tiles for community blocks (mfma_tile.hip) ----
// Tile t covers rows and columns [t*kWinRows, (t+1)*kWinRows).  Its dense
// fp16 values are stored in the operand order of v_mfma_f32_32x32x16_f16: for
// row group rg (32 rows) and k-step ks (16 columns), 64 lanes x 8 halves,
// lane l holding row rg*32 + l%32, columns ks*16 + 8*(l/32) .. +7.
struct MfmaArgs {
    const uint4 *atiles;   // [ntiles][8][kMfmaKSteps][64] x 8 fp16
    const int *rowptr;     // int32 [M+1] of the whole matrix (mean divisor)
    const int *rrowptr;    // int32 [M+1] residual CSR (entries outside the row's tile)
    const int *rcol;       // int32 [rnnz]
    const float *rval;     // fp32 [rnnz] or nullptr
    const float *B;        // fp32 [K, N]
    float *C;              // fp32 [M, N]
    int64_t M, K, N;
    int64_t nslices;       // kWinCols-wide column slices
    int mean;
    int xcd_remap;
};
hipError_t mfma_build_tiles(const int *rowptr, const int *col, const float *val, int64_t M, uint4 *atiles,
                            int64_t ntiles, int *rrowptr, int *range_flag, hipStream_t s);
hipError_t mfma_write_residual(const int *rowptr, const int *col, const float *val, int64_t M,
                               const int *rrowptr, int *rcol, float *rval, hipStream_t s);
hipError_t launch_mfma(const MfmaArgs &a, bool has_val, hipStream_t s);

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
hipError_t coo_to_csr(const int64_t *row, const int64_t *col, const float *val, int64_t E, int64_t M, int64_t K,
                      int64_t *rowptr_out, int64_t *col_out, float *val_out, int64_t *first_bad, hipStream_t s);
hipError_t transpose_csr(const int *rowptr, const int *col, const float *val, int64_t M, int64_t K, int64_t nnz,
                         bool scale, int64_t *rowptr_t, int64_t *col_t, float *val_t, hipStream_t s);
hipError_t launch_maxgrad(const MaxGradArgs &a, hipStream_t s);

}  // namespace gspmm

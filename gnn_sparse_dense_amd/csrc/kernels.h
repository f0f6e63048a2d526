// Device-side contract of the CSR SpMM kernels: tuning constants and the
// argument structs the kernels take.  Host-only declarations live in
// spmm_internal.h and plan.h.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

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
constexpr int kMergeItems = 512;        // merge-path items (entries + row ends) per wave
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
    // split tiles (fp32-level accuracy): A = (hi + lo) * 2^-tile_exp
    const uint4 *atiles_lo;  // same layout as atiles, or nullptr
    const int *tile_exp;     // int32 [ntiles]
};

// Arguments of the V = 2 panel kernel (pair_kernel.hip).
struct PairArgs {
    const int *prow;          // int32 [npanels+1]: vector range of each panel of rows 2g, 2g+1
    const unsigned *pcol;     // uint32 [nvec]: column | row-2g absent << 30 | row-2g+1 absent << 31
    const float *pval;        // fp32 [nvec][2] or nullptr
    const int *rowptr;        // int32 [M+1] (row degrees)
    const float *B;           // fp32 [K, N]
    float *C;                 // fp32 [M, N]
    int64_t *argmax;          // int64 [M, N] or nullptr
    int64_t M, N;
    int64_t npanels;          // panels: tasks end here
    int64_t task_base;        // first panel of this launch
    int mean;
    int xcd_remap;
};
typedef void (*PairKernelFn)(PairArgs);

// Arguments of the merge-path kernel and its fix-up (merge_kernel.hip).
struct MergeArgs {
    const int *rowptr;        // int32 [M+1]
    const int *col;           // int32 [nnz]
    const float *val;         // fp32 [nnz] or nullptr
    const int *seg_row;       // int32 [nseg+1]: row ends consumed before segment w
    const int *seg_entry;     // int32 [nseg+1]: entries consumed before segment w
    const float *B;           // fp32 [K, N]
    float *C;                 // fp32 [M, N]
    int64_t *argmax;          // int64 [M, N] or nullptr
    float *carry;             // fp32 [nseg, kPartialWidth]: open row's partial per segment
    int *carry_arg;           // int32 [nseg, kPartialWidth] (max)
    int *carry_row;           // int32 [nseg]: the open row, or -1
    int64_t M, N, nseg;
    int64_t c_begin, c_end;   // columns of this pass (at most kPartialWidth)
    int mean;
};
typedef void (*MergeKernelFn)(MergeArgs);

}  // namespace gspmm

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
constexpr int kXcdChunk = 256;           // consecutive blocks one XCD takes at a time
constexpr int kTileRows = 8;            // rows per row-tile record
constexpr int kTileLdsWords = 512;      // LDS words per wave for row-tile records (2 records)
constexpr int kTileMaxCap = 120;        // largest entries per row-tile record
constexpr int kWinRows = 256;           // rows of a community window
constexpr int kWinCols = 64;            // B columns staged per window block
constexpr int kWinBlock = 1024;         // threads of a window block
constexpr int kWinChunk = 128;          // staged entries per wave in window blocks

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
    const int *win_lo;     // int32 [M]: entries of row i below its window (sorted-row window kernel)
    const int *win_in;     // int32 [M]: entries of row i inside its window
    const int *task_perm;  // piece mode, or nullptr: task t computes piece task_perm[t]
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
    bool batch4;  // row tiles of 4 lanes x float4: entries in batches of 4 instead of 8
};

typedef void (*RowKernelFn)(RowArgs);

}  // namespace gspmm

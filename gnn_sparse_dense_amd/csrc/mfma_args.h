// Device-side contract of the matrix-core community tile kernel
// (mfma_tile.hip): constants and argument struct.
#pragma once

#include "kernels.h"

namespace gspmm {

constexpr int kMfmaKSteps = kWinRows / 16;   // k-steps of 16 per 256-wide community tile
constexpr int kMfmaBtPitch = kWinRows + 8;   // fp16 per staged B^T row of fp16 tiles (16-byte skew per row)

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

}  // namespace gspmm

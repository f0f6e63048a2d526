// Device-side contract of the merge-path kernel (merge_kernel.hip):
// constants and argument struct.
#pragma once

#include "kernels.h"

namespace gspmm {

constexpr int kMergeItems = 512;   // merge-path items (entries + row ends) per wave

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

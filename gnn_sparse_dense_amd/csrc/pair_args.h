// Device-side contract of the V = 2 panel kernel (pair_kernel.hip):
// argument struct.
#pragma once

#include "kernels.h"

namespace gspmm {

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

}  // namespace gspmm

// Ordered combine of split-row pieces.
//
// A row longer than the split threshold is cut into fixed-length pieces that
// run as independent tasks of the row kernel (ParamSpMM section 3.2: workload
// balancing splits a heavy row's entries across warps; graph-spmm card,
// "Requirements and limits": the card leaves the hubs of power-law graphs
// unbalanced under one warp per row).  The
// pages combine pieces with atomic adds; here each piece writes its own
// partial row and this kernel folds them in piece order, so the result does
// not depend on scheduling: sum = ((P0 + P1) + P2) + ..., max keeps the
// earlier piece on equal values (strict '>'), which preserves "first entry in
// stored order wins".  mean divides the folded sum by the row degree.
#include "spmm_internal.h"

namespace gspmm {

template <bool IS_MAX>
__global__ __launch_bounds__(kBlock) void combine_kernel(CombineArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t h = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (h >= a.n_heavy) return;
    const int row = a.heavy_rows[h];
    const int s0 = a.seg_first[h];
    const int s1 = a.seg_first[h + 1];
    const int deg = a.rowptr[row + 1] - a.rowptr[row];
    const int64_t width = a.c_end - a.c_begin;
    for (int64_t c = lane; c < width; c += 64) {
        float acc = a.partial[(int64_t)s0 * kPartialWidth + c];
        int arg = 0;
        if constexpr (IS_MAX) arg = a.part_arg[(int64_t)s0 * kPartialWidth + c];
        for (int s = s0 + 1; s < s1; ++s) {
            const float x = a.partial[(int64_t)s * kPartialWidth + c];
            if constexpr (IS_MAX) {
                const int ax = a.part_arg[(int64_t)s * kPartialWidth + c];
                if (x > acc) {
                    acc = x;
                    arg = ax;
                }
            } else {
                acc = acc + x;
            }
        }
        const int64_t o = (int64_t)row * a.N + a.c_begin + c;
        if constexpr (IS_MAX) {
            a.C[o] = acc;
            if (a.argmax) a.argmax[o] = arg;
        } else {
            a.C[o] = a.mean ? acc / (float)deg : acc;
        }
    }
}

hipError_t launch_combine(const CombineArgs &a, bool is_max, hipStream_t s) {
    if (a.n_heavy <= 0) return hipSuccess;
    const dim3 grid((unsigned)((a.n_heavy + kWaves - 1) / kWaves));
    if (is_max) hipLaunchKernelGGL(combine_kernel<true>, grid, dim3(kBlock), 0, s, a);
    else hipLaunchKernelGGL(combine_kernel<false>, grid, dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

RowKernelFn row_kernel(const RowKernelKey &k) {
    switch (k.vec) {
        case 1: return row_kernel_v1(k);
        case 2: return row_kernel_v2(k);
        case 4: return row_kernel_v4(k);
    }
    return nullptr;
}

}  // namespace gspmm

// Instantiations and launcher of the community-window kernels.
#include "row_kernel_impl.h"

namespace gspmm {

hipError_t launch_window(const RowArgs &a, bool has_val, bool is_max, bool sorted, hipStream_t s) {
    const int64_t ntiles = (a.ntasks + kWinRows - 1) / kWinRows;
    const int64_t slices = (a.N + kWinCols - 1) / kWinCols;
    if (ntiles <= 0) return hipSuccess;
    if (ntiles > (int64_t)(UINT32_MAX / kWinBlock) || slices > 65535) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)ntiles, (unsigned)slices);
    void (*fn)(RowArgs);
    if (sorted) {
        if (is_max) fn = has_val ? window_sorted_kernel_t<true, true> : window_sorted_kernel_t<false, true>;
        else fn = has_val ? window_sorted_kernel_t<true, false> : window_sorted_kernel_t<false, false>;
    } else {
        if (is_max) fn = has_val ? window_kernel_t<true, true> : window_kernel_t<false, true>;
        else fn = has_val ? window_kernel_t<true, false> : window_kernel_t<false, false>;
    }
    hipLaunchKernelGGL(fn, grid, dim3(kWinBlock), 0, s, a);
    return hipGetLastError();
}

}  // namespace gspmm

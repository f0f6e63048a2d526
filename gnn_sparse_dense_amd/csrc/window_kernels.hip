// Instantiations and launcher of the community-window kernel.
#include "row_kernel_impl.h"

namespace gspmm {

hipError_t launch_window(const RowArgs &a, bool has_val, bool is_max, hipStream_t s) {
    const int64_t ntiles = (a.ntasks + kWinRows - 1) / kWinRows;
    const int64_t slices = (a.N + kWinCols - 1) / kWinCols;
    if (ntiles <= 0) return hipSuccess;
    if (ntiles > (int64_t)(UINT32_MAX / kWinBlock) || slices > 65535) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)ntiles, (unsigned)slices);
    if (is_max) {
        if (has_val) hipLaunchKernelGGL((window_kernel_t<true, true>), grid, dim3(kWinBlock), 0, s, a);
        else hipLaunchKernelGGL((window_kernel_t<false, true>), grid, dim3(kWinBlock), 0, s, a);
    } else {
        if (has_val) hipLaunchKernelGGL((window_kernel_t<true, false>), grid, dim3(kWinBlock), 0, s, a);
        else hipLaunchKernelGGL((window_kernel_t<false, false>), grid, dim3(kWinBlock), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace gspmm

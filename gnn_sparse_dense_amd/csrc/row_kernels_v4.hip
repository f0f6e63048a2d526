// Row-kernel instantiations for 4-float lane accesses.
#include "row_kernel_impl.h"

namespace gspmm {

RowKernelFn row_kernel_v4(const RowKernelKey &k) { return pick_row_kernel_vec<4>(k); }

}  // namespace gspmm

// Row-kernel instantiations for 1-float lane accesses.
#include "row_kernel_impl.h"

namespace gspmm {

RowKernelFn row_kernel_v1(const RowKernelKey &k) { return pick_row_kernel_vec<1>(k); }

}  // namespace gspmm

// Row-kernel instantiations for 2-float lane accesses.
#include "row_kernel_impl.h"

namespace gspmm {

RowKernelFn row_kernel_v2(const RowKernelKey &k) { return pick_row_kernel_vec<2>(k); }

}  // namespace gspmm

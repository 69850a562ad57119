// Fused-stack kernel for windows of up to 16 rows.
#include "qgemv_kernels.h"

namespace qg {

StackFn stack_kernel_m16() { return qrow_stack<16>; }

}  // namespace qg

// Fused-stack kernel for windows of up to 2 rows.
#include "qgemv_kernels.h"

namespace qg {

StackFn stack_kernel_m2() { return qrow_stack<2>; }

}  // namespace qg

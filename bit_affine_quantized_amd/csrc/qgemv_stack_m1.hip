// Fused-stack kernel for windows of up to 1 row.
#include "qgemv_kernels.h"

namespace qg {

StackFn stack_kernel_m1() { return qrow_stack<1>; }

}  // namespace qg

// Fused-stack kernel for windows of up to 4 rows.
#include "qgemv_kernels.h"

namespace qg {

StackFn stack_kernel_m4() { return qrow_stack<4>; }

}  // namespace qg

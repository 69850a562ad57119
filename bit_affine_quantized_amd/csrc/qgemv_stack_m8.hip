// Fused-stack kernel for windows of up to 8 rows.
#include "qgemv_kernels.h"

namespace qg {

StackFn stack_kernel_m8() { return qrow_stack<8>; }

}  // namespace qg

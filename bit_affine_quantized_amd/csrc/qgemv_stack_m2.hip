// Fused-stack kernels (dot and matrix-core forms) for windows of up to 2 rows.
#include "qgemv_kernels.h"

namespace qg {

StackKernels stack_kernels_m2() { return {qrow_stack<2>, qrow_stack_mfma<2>}; }

}  // namespace qg

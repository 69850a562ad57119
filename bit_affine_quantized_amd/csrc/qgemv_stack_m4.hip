// Fused-stack kernels (dot and matrix-core forms) for windows of up to 4 rows.
#include "qgemv_kernels.h"

namespace qg {

StackKernels stack_kernels_m4() { return {qrow_stack<4>, qrow_stack_mfma<4>}; }

}  // namespace qg

// Fused-stack kernels (dot and matrix-core forms) for one-row windows.
#include "qgemv_kernels.h"

namespace qg {

StackKernels stack_kernels_m1() { return {qrow_stack<1>, qrow_stack_mfma<1>}; }

}  // namespace qg

// Fused-stack kernels (dot and matrix-core forms) for windows of up to 16 rows.
#include "qgemv_kernels.h"

namespace qg {

StackKernels stack_kernels_m16() { return {qrow_stack<16>, qrow_stack_mfma<16>}; }

}  // namespace qg

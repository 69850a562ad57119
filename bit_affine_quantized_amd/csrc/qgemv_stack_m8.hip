// Fused-stack kernels (dot and matrix-core forms) for windows of up to 8 rows.
#include "qgemv_kernels.h"

namespace qg {

StackKernels stack_kernels_m8() { return {qrow_stack<8>, qrow_stack_mfma<8>}; }

}  // namespace qg

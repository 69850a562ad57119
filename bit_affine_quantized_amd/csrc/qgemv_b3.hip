// Kernels of the 3-bit code width, groups of 32, 64 and 128.
#include "qgemv_kernels.h"

namespace qg {

const Entry* entries_b3() {
  static const Entry table[3] = {make_entry<3, 32>(), make_entry<3, 64>(), make_entry<3, 128>()};
  return table;
}

}  // namespace qg

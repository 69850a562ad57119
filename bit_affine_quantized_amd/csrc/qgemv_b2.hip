// Kernels of the 2-bit code width, groups of 32, 64 and 128.
#include "qgemv_kernels.h"

namespace qg {

const Entry* entries_b2() {
  static const Entry table[3] = {make_entry<2, 32>(), make_entry<2, 64>(), make_entry<2, 128>()};
  return table;
}

}  // namespace qg

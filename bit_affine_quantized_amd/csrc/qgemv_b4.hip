// Kernels of the 4-bit code width, groups of 32, 64 and 128.
#include "qgemv_kernels.h"

namespace qg {

const Entry* entries_b4() {
  static const Entry table[3] = {make_entry<4, 32>(), make_entry<4, 64>(), make_entry<4, 128>()};
  return table;
}

}  // namespace qg

// Kernels of the 6-bit code width, groups of 32, 64 and 128.
#include "qgemv_kernels.h"

namespace qg {

const Entry* entries_b6() {
  static const Entry table[3] = {make_entry<6, 32>(), make_entry<6, 64>(), make_entry<6, 128>()};
  return table;
}

}  // namespace qg

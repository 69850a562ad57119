// Kernels of the 5-bit code width, groups of 32, 64 and 128.
#include "qgemv_kernels.h"

namespace qg {

const Entry* entries_b5() {
  static const Entry table[3] = {make_entry<5, 32>(), make_entry<5, 64>(), make_entry<5, 128>()};
  return table;
}

}  // namespace qg

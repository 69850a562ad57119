// Kernels of the 8-bit code width, groups of 32, 64 and 128.
#include "qgemv_kernels.h"

namespace qg {

const Entry* entries_b8() {
  static const Entry table[3] = {make_entry<8, 32>(), make_entry<8, 64>(), make_entry<8, 128>()};
  return table;
}

}  // namespace qg

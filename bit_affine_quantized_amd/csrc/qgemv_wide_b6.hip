// Wide-window matrix-core kernels of the 6-bit code width, groups of 32, 64 and 128.
#include "qgemv_kernels.h"

namespace qg {

const WideEntry* wide_entries_b6() {
  static const WideEntry table[3] = {make_wide_entry<6, 32>(), make_wide_entry<6, 64>(), make_wide_entry<6, 128>()};
  return table;
}

}  // namespace qg

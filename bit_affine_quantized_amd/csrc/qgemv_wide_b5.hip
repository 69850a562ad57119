// Wide-window matrix-core kernels of the 5-bit code width, groups of 32, 64 and 128.
#include "qgemv_kernels.h"

namespace qg {

const WideEntry* wide_entries_b5() {
  static const WideEntry table[3] = {make_wide_entry<5, 32>(), make_wide_entry<5, 64>(), make_wide_entry<5, 128>()};
  return table;
}

}  // namespace qg

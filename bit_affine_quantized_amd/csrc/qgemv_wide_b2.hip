// Wide-window matrix-core kernels of the 2-bit code width, groups of 32, 64 and 128.
#include "qgemv_kernels.h"

namespace qg {

const WideEntry* wide_entries_b2() {
  static const WideEntry table[3] = {make_wide_entry<2, 32>(), make_wide_entry<2, 64>(), make_wide_entry<2, 128>()};
  return table;
}

}  // namespace qg

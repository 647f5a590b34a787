// skg_valu_ga.hip -- VALU kernel instantiations for M = 1..8, activation
// chunks loaded from global memory in the load ring.
#include "skg_device.h"

namespace skg {

KernelPtr valu_kernel_ga(int M, int variant) {
    static const KernelPtr table[8][kNumValu] = {
        SKG_VALU_ROW_GA(1), SKG_VALU_ROW_GA(2), SKG_VALU_ROW_GA(3), SKG_VALU_ROW_GA(4),
        SKG_VALU_ROW_GA(5), SKG_VALU_ROW_GA(6), SKG_VALU_ROW_GA(7), SKG_VALU_ROW_GA(8)};
    if (M < 1 || M > 8 || variant < 0 || variant >= kNumValu) return nullptr;
    return table[M - 1][variant];
}

}  // namespace skg

// skg_valu_ga.hip -- VALU kernel instantiations for M = 1..8, activation
// chunks loaded from global memory in the load ring.
#include "skg_device.h"

namespace skg {

KernelPtr valu_kernel_ga(int M, int variant) {
    static const KernelPtr table[8][kNumValu] = {
        SKG_VALU_ROW(1, true), SKG_VALU_ROW(2, true), SKG_VALU_ROW(3, true),
        SKG_VALU_ROW(4, true), SKG_VALU_ROW(5, true), SKG_VALU_ROW(6, true),
        SKG_VALU_ROW(7, true), SKG_VALU_ROW(8, true)};
    if (M < 1 || M > 8 || variant < 0 || variant >= kNumValu) return nullptr;
    return table[M - 1][variant];
}

}  // namespace skg

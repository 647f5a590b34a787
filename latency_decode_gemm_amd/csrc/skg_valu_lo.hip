// skg_valu_lo.hip -- VALU kernel instantiations for M = 1..8.
#include "skg_device.h"

namespace skg {

KernelPtr valu_kernel_lo(int M, int variant) {
    static const KernelPtr table[8][kNumValu] = {
        SKG_VALU_ROW(1), SKG_VALU_ROW(2), SKG_VALU_ROW(3), SKG_VALU_ROW(4),
        SKG_VALU_ROW(5), SKG_VALU_ROW(6), SKG_VALU_ROW(7), SKG_VALU_ROW(8)};
    if (M < 1 || M > 8 || variant < 0 || variant >= kNumValu) return nullptr;
    return table[M - 1][variant];
}

}  // namespace skg

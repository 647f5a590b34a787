// skg_valu_lo.hip -- VALU kernel instantiations for M = 1..8, A staged in LDS.
#include "skg_device.h"

namespace skg {

KernelPtr valu_kernel_lo(int M, int variant) {
    static const KernelPtr table[8][kNumValu] = {
        SKG_VALU_ROW(1, false), SKG_VALU_ROW(2, false), SKG_VALU_ROW(3, false),
        SKG_VALU_ROW(4, false), SKG_VALU_ROW(5, false), SKG_VALU_ROW(6, false),
        SKG_VALU_ROW(7, false), SKG_VALU_ROW(8, false)};
    if (M < 1 || M > 8 || variant < 0 || variant >= kNumValu) return nullptr;
    return table[M - 1][variant];
}

}  // namespace skg

// skg_valu_hi.hip -- VALU kernel instantiations for M = 9..16, A staged in LDS.
#include "skg_device.h"

namespace skg {

KernelPtr valu_kernel_hi(int M, int variant) {
    static const KernelPtr table[8][kNumValu] = {
        SKG_VALU_ROW(9, false), SKG_VALU_ROW(10, false), SKG_VALU_ROW(11, false),
        SKG_VALU_ROW(12, false), SKG_VALU_ROW(13, false), SKG_VALU_ROW(14, false),
        SKG_VALU_ROW(15, false), SKG_VALU_ROW(16, false)};
    if (M < 9 || M > 16 || variant < 0 || variant >= kNumValu) return nullptr;
    return table[M - 9][variant];
}

}  // namespace skg

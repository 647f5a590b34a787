// skg_f32w_ga.hip -- VALU kernel instantiations over fp32 weights for
// M = 1..8, activation chunks loaded from global memory in the load ring.
#include "skg_device.h"

namespace skg {

KernelPtr valu_kernel_f32w_ga(int M, int variant) {
    static const KernelPtr table[8][kNumValu] = {
        SKG_VALU_ROW_F32W(1, true), SKG_VALU_ROW_F32W(2, true), SKG_VALU_ROW_F32W(3, true),
        SKG_VALU_ROW_F32W(4, true), SKG_VALU_ROW_F32W(5, true), SKG_VALU_ROW_F32W(6, true),
        SKG_VALU_ROW_F32W(7, true), SKG_VALU_ROW_F32W(8, true)};
    if (M < 1 || M > 8 || variant < 0 || variant >= kNumValu) return nullptr;
    return table[M - 1][variant];
}

}  // namespace skg

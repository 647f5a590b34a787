// skg_f32w_lo.hip -- VALU kernel instantiations over fp32 weights for
// M = 1..8, A staged in LDS.
#include "skg_device.h"

namespace skg {

KernelPtr valu_kernel_f32w_lo(int M, int variant) {
    static const KernelPtr table[8][kNumValu] = {
        SKG_VALU_ROW_F32W(1, false), SKG_VALU_ROW_F32W(2, false), SKG_VALU_ROW_F32W(3, false),
        SKG_VALU_ROW_F32W(4, false), SKG_VALU_ROW_F32W(5, false), SKG_VALU_ROW_F32W(6, false),
        SKG_VALU_ROW_F32W(7, false), SKG_VALU_ROW_F32W(8, false)};
    if (M < 1 || M > 8 || variant < 0 || variant >= kNumValu) return nullptr;
    return table[M - 1][variant];
}

}  // namespace skg

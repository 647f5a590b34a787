// skg_f32w_hi.hip -- VALU kernel instantiations over fp32 weights for
// M = 9..16, A staged in LDS.
#include "skg_device.h"

namespace skg {

KernelPtr valu_kernel_f32w_hi(int M, int variant) {
    static const KernelPtr table[8][kNumValu] = {
        SKG_VALU_ROW_F32W(9, false), SKG_VALU_ROW_F32W(10, false), SKG_VALU_ROW_F32W(11, false),
        SKG_VALU_ROW_F32W(12, false), SKG_VALU_ROW_F32W(13, false), SKG_VALU_ROW_F32W(14, false),
        SKG_VALU_ROW_F32W(15, false), SKG_VALU_ROW_F32W(16, false)};
    if (M < 9 || M > 16 || variant < 0 || variant >= kNumValu) return nullptr;
    return table[M - 9][variant];
}

}  // namespace skg

// skg_mfma_mt4.hip -- MFMA kernels for M = 49..64 (4 token tiles of 16).
#include "skg_mfma_mid.h"

namespace skg {

KernelPtr mfma_kernel_mt4(int inner, int row_tiles, int depth) {
    static const MidRow rows[] = SKG_MID_TABLE(4);
    return mid_lookup(rows, (int)(sizeof(rows) / sizeof(rows[0])), inner, row_tiles, depth);
}

}  // namespace skg

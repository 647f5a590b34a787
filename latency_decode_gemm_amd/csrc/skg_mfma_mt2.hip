// skg_mfma_mt2.hip -- MFMA kernels for M = 17..32 (2 token tiles of 16).
#include "skg_mfma_mid.h"

namespace skg {

KernelPtr mfma_kernel_mt2(int inner, int row_tiles, int depth) {
    static const MidRow rows[] = SKG_MID_TABLE(2);
    return mid_lookup(rows, (int)(sizeof(rows) / sizeof(rows[0])), inner, row_tiles, depth);
}

}  // namespace skg

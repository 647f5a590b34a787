// skg_mfma_mt3.hip -- MFMA kernels for M = 33..48 (3 token tiles of 16).
#include "skg_mfma_mid.h"

namespace skg {

KernelPtr mfma_kernel_mt3(int inner, int row_tiles, int depth) {
    static const MidRow rows[] = SKG_MID_TABLE(3);
    return mid_lookup(rows, (int)(sizeof(rows) / sizeof(rows[0])), inner, row_tiles, depth);
}

}  // namespace skg

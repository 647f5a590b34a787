// skg_mfma_sync.hip -- the LDS-ring matrix-core kernel with its waves meeting
// at a barrier every K step (SKG_INNER_MFMA_RING_SYNC) and with the step's
// activation tile shared by the workgroup's waves (SKG_INNER_MFMA_RING_SHARED),
// M <= 16, activations loaded per step.  Row tiles 1 and 2 with the depths of
// the other matrix-core kinds; the shared ring needs depth >= 3.
#include "skg_device.h"

namespace skg {
namespace {

template <int G, int PF, int AQ, int SY>
constexpr KernelPtr sync_kernel() {
    if constexpr (SY == 2 && PF < 3)
        return nullptr;
    else
        return skg_mfma_ring_kernel<G, PF, AQ, 1, SY>;
}

struct SyncRow {
    int G, PF;
    KernelPtr k[2][2];  // [SY - 1][AQ == 4]
};
#define SKG_SYNC_ROW(G, PF)                                                              \
    {G,                                                                                  \
     PF,                                                                                 \
     {{sync_kernel<G, PF, 2, 1>(), sync_kernel<G, PF, 4, 1>()},                          \
      {sync_kernel<G, PF, 2, 2>(), sync_kernel<G, PF, 4, 2>()}}}
const SyncRow kSyncRows[] = {SKG_SYNC_ROW(1, 2), SKG_SYNC_ROW(1, 3), SKG_SYNC_ROW(1, 4),
                             SKG_SYNC_ROW(1, 6), SKG_SYNC_ROW(2, 1), SKG_SYNC_ROW(2, 2),
                             SKG_SYNC_ROW(2, 3), SKG_SYNC_ROW(2, 4)};
#undef SKG_SYNC_ROW

}  // namespace

KernelPtr mfma_kernel_sync(int inner, int M, int row_tiles, int depth) {
    if (M < 1 || M > 16) return nullptr;
    const int sy = inner == SKG_INNER_MFMA_RING_SYNC ? 1 : inner == SKG_INNER_MFMA_RING_SHARED ? 2 : 0;
    if (!sy) return nullptr;
    for (const SyncRow &r : kSyncRows)
        if (r.G == row_tiles && r.PF == depth) return r.k[sy - 1][M > 8 ? 1 : 0];
    return nullptr;
}

}  // namespace skg

// skg_mfma_mid.h -- instantiation of the MFMA kernels for 16 < M <= 64: MT
// token tiles of 16 (MT = 2, 3, 4), included by skg_mfma_mt2/3/4.hip.
//
// A combination is built only where it fits, as measured with the
// compiler's resource-usage report (no scratch): with the load ring in LDS,
// the ring's loads stay within the wave's counter of outstanding vector
// memory operations (depth x loads per step < 64) and the operands of one
// step, read ahead of its MFMAs, stay in registers (row tiles x token tiles
// <= 6); with the ring in registers, its 16-byte slots plus the accumulators
// take at most 176 VGPRs.  The rest are nullptr and no configuration
// reaches them.
#pragma once

#include "skg_device.h"

namespace skg {
namespace {

template <int G, int PF, int MT, bool RING, bool AG>
constexpr bool mid_builds() {
    constexpr int loads = 4 * G + (AG ? 4 * MT : 0);  // 16-byte loads per K step
    return RING ? (PF * loads < 64 && G * MT <= 6) : (4 * PF * loads + 4 * G * MT <= 176);
}

template <int G, int PF, int MT, bool RING, bool AG>
constexpr KernelPtr mid_kernel() {
    if constexpr (!mid_builds<G, PF, MT, RING, AG>())
        return nullptr;
    else if constexpr (RING)
        return skg_mfma_ring_kernel<G, PF, AG ? 4 : 0, MT>;
    else
        return skg_mfma_kernel<G, PF, AG ? 4 : 0, MT>;
}

// Per (G, PF): the four inner kinds in the order MFMA, MFMA_GA, MFMA_RING,
// MFMA_RING_GA.
struct MidRow {
    int G, PF;
    KernelPtr k[4];
};

#define SKG_MID(G, PF, MT)                                                                 \
    {G, PF, {mid_kernel<G, PF, MT, false, false>(), mid_kernel<G, PF, MT, false, true>(), \
             mid_kernel<G, PF, MT, true, false>(), mid_kernel<G, PF, MT, true, true>()}}
// the (G, PF) pairs of the 16-token kernels
#define SKG_MID_TABLE(MT)                                                                  \
    {SKG_MID(1, 2, MT), SKG_MID(1, 3, MT), SKG_MID(1, 4, MT), SKG_MID(1, 6, MT),          \
     SKG_MID(2, 1, MT), SKG_MID(2, 2, MT), SKG_MID(2, 3, MT), SKG_MID(2, 4, MT),          \
     SKG_MID(4, 1, MT), SKG_MID(4, 2, MT)}

inline KernelPtr mid_lookup(const MidRow *rows, int n, int inner, int G, int PF) {
    const int kind = inner == SKG_INNER_MFMA           ? 0
                     : inner == SKG_INNER_MFMA_GA      ? 1
                     : inner == SKG_INNER_MFMA_RING    ? 2
                     : inner == SKG_INNER_MFMA_RING_GA ? 3
                                                       : -1;
    if (kind < 0) return nullptr;
    for (int i = 0; i < n; ++i)
        if (rows[i].G == G && rows[i].PF == PF) return rows[i].k[kind];
    return nullptr;
}

}  // namespace
}  // namespace skg

// Internal interface between the C-ABI layer (skg_api.cpp) and the gfx950
// kernels (skg_device.h, instantiated in skg_valu_lo.hip, skg_valu_hi.hip and
// skg_launch.hip).  Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/skinny_gemm.h"

namespace skg {

// K is walked in chunks of 8 bf16 (one 16-byte load).
constexpr int kChunk = 8;
// K-step of one wave, in chunks (both kernels): 16 lanes x 1 chunk = 128 k;
// the MFMA kernel runs four 16x16x32 instructions per step.
constexpr int kValuStep = 16;
// gfx950 LDS per workgroup.
constexpr int kMaxLdsBytes = 160 * 1024;
constexpr int kMaxWaves = 8;  // 512 threads: up to 256 VGPRs per lane
// SKG_BACKEND_EVEN: workgroups per rb_per_wg (the CU count of MI355X)
constexpr int kEvenUnit = 256;
// Largest K and N a configuration takes (the launch geometry stays in int).
constexpr int kMaxK = 1 << 28;
constexpr int kMaxN = 1 << 30;

// Everything a kernel needs, passed by value.
struct KParams {
    const uint16_t *A;
    const uint16_t *B;
    void *C;
    float *ws;                 // two-pass split-K partials [num_rb][split_k][M][rows_per_wg]
    unsigned long long *slots; // one-pass split-K tree slots [num_rb][split_k - 1][M][rows_per_wg],
                               // zero between calls
    int64_t lda, ldb, ldc;
    int M, N, K;
    int out_bf16;
    int nck;          // ceil(K / 8)
    int nfull;        // K / 8 (chunks with all 8 elements inside K)
    int split_k;      // workgroups along K per row block
    int two_pass;     // split-K partials are summed by a second kernel
    int even;         // SKG_BACKEND_EVEN: row block rb is rows [rb N / num_rb, (rb + 1) N / num_rb)
    int even_q, even_r; // N = even_q num_rb + even_r (SKG_BACKEND_EVEN)
    int wg_chunks;    // chunks per split (multiple of wave_chunks)
    int wave_chunks;  // chunks per K-wave (multiple of the K-step)
    int waves_n, waves_k; // the workgroup's waves (64 * waves_n * waves_k threads)
    int rows_per_wg;
    int num_rb;
    int grid_rb;      // workgroups per K slice (the grid is grid_rb x split_k)
    int lds_stride;   // bf16 elements per staged A row in LDS
    int stash_offset; // byte offset in LDS of the per-row-block partial sums
                      // that the epilogue combines
    int tr_offset;    // byte offset of the MFMA kernel's per-wave transpose tiles
    int w_f32;        // B holds fp32 weights (rows of ldb fp32 elements)
};

// Derived launch geometry for (M, K, N, cfg).
struct Geometry {
    int step;          // K-step in chunks
    int nck, nfull;
    int wave_chunks, wg_chunks;
    int rows_per_wave, rows_per_wg, num_rb;
    int grid_rb;       // workgroups per K slice (each takes every grid_rb-th row block)
    int threads;
    int lds_stride;    // elements
    size_t lds_bytes;
    int stash_offset, tr_offset;
    size_t ws_floats;   // two-pass split-K partial floats
    size_t slot_words;  // one-pass split-K tree slots, in 32-bit words (zero between calls)
};

// Fills g; returns false if cfg cannot run (M, K, N).
bool make_geometry(int M, int K, int N, const skg_config &cfg, Geometry *g);

// Whether (inner, row_tiles, depth) has a compiled kernel (f32w: one over fp32
// weights for M tokens; those exist for the VALU kinds only, and not for
// every M).
bool variant_exists(int inner, int row_tiles, int depth, bool f32w = false, int M = 1);

// Enqueues the kernel for p (p.w_f32 selects the fp32-weight kernels) with
// geometry g on stream.  Non-null start/stop
// events are recorded by the dispatch itself (kernel start and end).
hipError_t launch(const KParams &p, const Geometry &g, const skg_config &cfg,
                  hipStream_t stream, hipEvent_t start = nullptr, hipEvent_t stop = nullptr);

// Zero-fills C[m*ldc + n] for K == 0.
hipError_t launch_zero_fill(void *C, int M, int N, int64_t ldc, int out_bf16,
                            hipStream_t stream, hipEvent_t start = nullptr,
                            hipEvent_t stop = nullptr);

// K in 1..7: one thread per output, plain fp32 sum (p needs A, B, C, lda,
// ldb, ldc, M, N, K, out_bf16, w_f32).
hipError_t launch_small_k(const KParams &p, hipStream_t stream, hipEvent_t start = nullptr,
                          hipEvent_t stop = nullptr);

// Streaming-read probe: 512 x 256 threads fold `n16` 16-byte words into sink[512].
constexpr int kReadProbeGrid = 512;
hipError_t launch_stream_read(const void *src, size_t n16, void *sink, hipStream_t stream);

// Loads a kernel's code object (forces lazy loading) for availability checks.
hipError_t probe_kernels();

// Static split-K scratch of the no-allocation entry point (skg_scratch.hip):
// kScratchSlotWords 32-bit words of tree slots (zero between calls), then
// kScratchPartialFloats fp32 partials, one array per device.
constexpr int kScratchSlotWords = SKG_SCRATCH_SLOT_BYTES / 4;
constexpr int kScratchPartialFloats = SKG_SCRATCH_PARTIAL_BYTES / 4;
constexpr int kScratchWords = kScratchSlotWords + kScratchPartialFloats;
// This device's scratch address (looked up once per device, with the device
// current; the slots are cleared on `stream` at that first use).
hipError_t static_scratch(hipStream_t stream, void **ptr);

// MFMA transpose tile per wave and 16-row tile: 16 rows x 16 chunks x 16 B.
constexpr int kTileBytes = 4096;

// Kernel variants.  VALU (row_tiles R, depth PF) pairs, in table order; the
// instantiations live in skg_valu_lo.hip (M = 1..8), skg_valu_hi.hip
// (M = 9..16) and skg_valu_ga.hip (activations from global memory, M = 1..8),
// the MFMA ones in skg_launch.hip.
using KernelPtr = void (*)(KParams);
constexpr int kValuVariants[][2] = {{1, 4}, {1, 8}, {1, 12}, {2, 2},
                                     {2, 4}, {2, 8}, {4, 2}, {4, 4}};
constexpr int kNumValu = sizeof(kValuVariants) / sizeof(kValuVariants[0]);
KernelPtr valu_kernel_lo(int M, int variant);
KernelPtr valu_kernel_hi(int M, int variant);
KernelPtr valu_kernel_ga(int M, int variant);  // activations from global memory, M <= 8
// MFMA kernels for 16 < M <= 64 (skg_mfma_mt2/3/4.hip: 2, 3, 4 token tiles
// of 16); nullptr where a combination is not built
KernelPtr mfma_kernel_mt2(int inner, int row_tiles, int depth);
KernelPtr mfma_kernel_mt3(int inner, int row_tiles, int depth);
KernelPtr mfma_kernel_mt4(int inner, int row_tiles, int depth);
// LDS-ring kernels with a barrier every K step, M <= 16 (skg_mfma_sync.hip);
// nullptr for other kinds or where a combination is not built
KernelPtr mfma_kernel_sync(int inner, int M, int row_tiles, int depth);
// tokens the VALU kernels (and so the fp32-weight path) take at most
constexpr int kMaxMValu = 16;
// the same three tables over fp32 weights (skg_f32w_lo/hi/ga.hip)
KernelPtr valu_kernel_f32w_lo(int M, int variant);
KernelPtr valu_kernel_f32w_hi(int M, int variant);
KernelPtr valu_kernel_f32w_ga(int M, int variant);

}  // namespace skg

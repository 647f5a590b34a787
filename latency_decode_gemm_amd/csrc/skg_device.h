// skg_device.h -- gfx950 kernels for C[M,N] = A[M,K] . B[N,K]^T, M <= 16.
//
// What is computed follows the PR #42562 page ("Add generic cuteDSL LL BF16
// router (GEMM)"): section 实现拆解 item 1 and the _ll_bf16_dotprod.py excerpt
// (each weight tile is loaded once with 128-bit loads, widened, and multiplied
// into one fp32 accumulator per token m; partial sums are reduced across lanes
// and through shared memory) and item 2 (K is split across several blocks
// whose partial sums are combined).  The kernels below are designed for CDNA4,
// not translated from that design:
//
//  * One launch streams B exactly once.  Rows of B are grouped in row blocks
//    of rows_per_wg rows; K is cut into split_k slices.  A workgroup owns one
//    K slice and a strided set of row blocks (blockIdx / split_k, then every
//    gridDim / split_k-th), so it stages A[:, slice] in LDS once (zero beyond
//    K) and then streams all of its row blocks.  Its waves split the rows of a
//    block (waves_n) and the slice (waves_k, equal parts).
//  * Every wave runs one flat stream of K steps over all its row blocks, with
//    `depth` steps of B loads in flight in a register ring; the loads of the
//    next row block are already in flight while the current block is reduced
//    and written.  Barriers inside that stream wait for LDS traffic only, so
//    they never drain the ring.
//  * VALU inner product: 16 lanes per row of B, so one 64-lane dwordx4 load
//    covers 4 rows x 256 contiguous bytes; products by v_dot2c_f32_bf16 (two
//    bf16 products added into fp32).  The 16 lanes of a row are combined with
//    a DPP reduce-scatter (row_mirror, row_half_mirror, quad_perm) that leaves
//    lane i of the row group with the sum for token m = i.
//  * MFMA inner product (v_mfma_f32_16x16x32_bf16): the activations are the
//    16-row operand (rows m >= M are zero), 16 rows of B are the 16 columns;
//    the instruction performs the K reduction, so no cross-lane step remains.
//  * Cross-wave (waves_k > 1): partials go through LDS (double-buffered per
//    row block) and wave 0 adds them in wave order.  Cross-workgroup
//    (split_k > 1): each workgroup stores its fp32 partial tile with
//    agent-scope atomic stores, waits for them, and takes a ticket with one
//    agent-scope atomic add; the workgroup that draws the last ticket reads the
//    split_k partials with agent-scope atomic loads, adds them in split order,
//    writes C and resets the ticket.  These accesses are coherent across the
//    XCDs' L2s without any L2 write-back or invalidate.  Nothing waits for
//    another workgroup, and no summation order depends on timing, so results
//    are bit-reproducible.
//  * Epilogue: fp32 stores, or bf16 round-to-nearest-even, at C[m*ldc + n];
//    other bytes of C are never written.
#pragma once

#include "skg_internal.h"

namespace skg {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ldg16(const uint16_t *p) {
    return *reinterpret_cast<const uint4 *>(p);
}

// Weight loads: every byte of B is read once, so they are marked
// non-temporal (streaming) and do not displace A from the caches.
__device__ __forceinline__ uint4 ldg16_stream(const uint16_t *p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint4 lds16(const uint16_t *p) {
    return *reinterpret_cast<const uint4 *>(p);
}

__device__ __forceinline__ void sts16(uint16_t *p, uint4 v) {
    *reinterpret_cast<uint4 *>(p) = v;
}

// Direct global -> LDS load of 16 bytes per lane (global_load_lds_dwordx4):
// lane l's 16 bytes from gsrc land at lds_base + 16 * l (lds_base is the same
// for the whole wave).  No VGPRs are used, so every staging load of a
// workgroup can be in flight at once; the data is in LDS once vmcnt drains.
__device__ __forceinline__ void lds_dma16(const uint16_t *gsrc, void *lds_base) {
    typedef const __attribute__((address_space(1))) void *gptr_t;
    typedef __attribute__((address_space(3))) void *lptr_t;
    __builtin_amdgcn_global_load_lds((gptr_t)(gsrc), (lptr_t)(lds_base), 16, 0, 0);
}

// Workgroup barrier that orders LDS accesses only: outstanding global loads
// stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Eight bf16 products accumulated into c, two per v_dot2c_f32_bf16.
__device__ __forceinline__ float dot8(const uint4 &a, const uint4 &b, float c) {
    c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.x),
                                        __builtin_bit_cast(bf16x2_t, b.x), c, false);
    c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.y),
                                        __builtin_bit_cast(bf16x2_t, b.y), c, false);
    c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.z),
                                        __builtin_bit_cast(bf16x2_t, b.z), c, false);
    c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.w),
                                        __builtin_bit_cast(bf16x2_t, b.w), c, false);
    return c;
}

// fp32 -> bf16, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ void store_c(const KParams &p, int m, int n, float v) {
    const int64_t off = (int64_t)m * p.ldc + n;
    if (p.out_bf16)
        reinterpret_cast<uint16_t *>(p.C)[off] = f32_to_bf16_rne(v);
    else
        reinterpret_cast<float *>(p.C)[off] = v;
}

// One 8-element chunk (k = 8c .. 8c+7) of the row starting at rowp, with
// every element at k >= K read as zero (no access beyond K).
template <bool STREAM = false>
__device__ __forceinline__ uint4 load_chunk_masked(const uint16_t *rowp, int c, const KParams &p) {
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (c < p.nfull) {
        v = STREAM ? ldg16_stream(rowp + (int64_t)c * kChunk) : ldg16(rowp + (int64_t)c * kChunk);
    } else if (c < p.nck) {
        // the one chunk that straddles K (K % 8 != 0)
        uint32_t w[4] = {0u, 0u, 0u, 0u};
        const int k0 = c * kChunk;
#pragma unroll
        for (int e = 0; e < kChunk; ++e) {
            if (k0 + e < p.K) {
                const uint32_t h = rowp[k0 + e];
                w[e >> 1] |= h << (16 * (e & 1));
            }
        }
        v = make_uint4(w[0], w[1], w[2], w[3]);
    }
    return v;
}

// Stage A[m, 8*wg_c0 : 8*(wg_c0 + wg_chunks)) for m < M into LDS rows of
// p.lds_stride elements; zeros beyond K.  Each wave moves blocks of 64 chunks
// (1 KB, one row) straight into LDS; the chunk straddling K and the chunks
// beyond it are written as (partial) zeros by ordinary LDS stores.  The
// caller's barrier waits for all of it.
__device__ __forceinline__ void stage_a(const KParams &p, uint16_t *As, int wg_c0) {
    const int lane = threadIdx.x & 63;
    const int nwaves = blockDim.x >> 6;
    const int nch = p.wg_chunks;
    const int nblk = (nch + 63) >> 6;  // 64-chunk blocks per row
    for (int blk = threadIdx.x >> 6; blk < p.M * nblk; blk += nwaves) {
        const int m = blk / nblk;
        const int cc0 = (blk - m * nblk) << 6;
        const int cc = cc0 + lane;
        const int c = wg_c0 + cc;
        const uint16_t *rowp = p.A + (int64_t)m * p.lda;
        uint16_t *dst = As + m * p.lds_stride + cc0 * kChunk;
        if (cc < nch) {
            if (c < p.nfull)
                lds_dma16(rowp + (int64_t)c * kChunk, dst);
            else
                sts16(dst + lane * kChunk, load_chunk_masked(rowp, c, p));
        }
    }
}

// ---- 16-lane DPP reduce-scatter --------------------------------------------
// dpp controls on gfx9: row_mirror (lane i <- 15-i), row_half_mirror
// (i <- 7-i within 8), quad_perm [2,3,0,1] (i <- i^2), quad_perm [1,0,3,2]
// (i <- i^1).  Each pairs lanes that differ in one bit of the lane index.
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppXor1 = 0xB1;

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Every lane adds its partner's copy: both end with the pair sum.
template <int CTRL, int NV>
__device__ __forceinline__ void butterfly_step(float *v) {
#pragma unroll
    for (int j = 0; j < NV; ++j) v[j] += dpp_f<CTRL>(v[j]);
}

// Halving step: the lane with the index bit BIT clear keeps values [0, H),
// the other keeps [H, 2H) (re-indexed to [0, H)), each adding the partner's
// copy of what it keeps.
template <int CTRL, int BIT, int H>
__device__ __forceinline__ void scatter_step(float *v, int lane) {
    const bool upper = (lane & BIT) != 0;
#pragma unroll
    for (int j = 0; j < H; ++j) {
        const float keep = upper ? v[j + H] : v[j];
        const float send = upper ? v[j] : v[j + H];
        v[j] = keep + dpp_f<CTRL>(send);
    }
}

// v[0..VP) per lane -> v[0] = sum over the 16 lanes of the row group of the
// value with index (lane & (VP - 1)).
template <int VP>
__device__ __forceinline__ void reduce16(float *v, int lane) {
    if constexpr (VP == 16) {
        scatter_step<kDppRowMirror, 8, 8>(v, lane);
        scatter_step<kDppRowHalfMirror, 4, 4>(v, lane);
        scatter_step<kDppXor2, 2, 2>(v, lane);
        scatter_step<kDppXor1, 1, 1>(v, lane);
    } else if constexpr (VP == 8) {
        butterfly_step<kDppRowMirror, 8>(v);
        scatter_step<kDppRowHalfMirror, 4, 4>(v, lane);
        scatter_step<kDppXor2, 2, 2>(v, lane);
        scatter_step<kDppXor1, 1, 1>(v, lane);
    } else if constexpr (VP == 4) {
        butterfly_step<kDppRowMirror, 4>(v);
        butterfly_step<kDppRowHalfMirror, 4>(v);
        scatter_step<kDppXor2, 2, 2>(v, lane);
        scatter_step<kDppXor1, 1, 1>(v, lane);
    } else if constexpr (VP == 2) {
        butterfly_step<kDppRowMirror, 2>(v);
        butterfly_step<kDppRowHalfMirror, 2>(v);
        butterfly_step<kDppXor2, 2>(v);
        scatter_step<kDppXor1, 1, 1>(v, lane);
    } else {
        butterfly_step<kDppRowMirror, 1>(v);
        butterfly_step<kDppRowHalfMirror, 1>(v);
        butterfly_step<kDppXor2, 1>(v);
        butterfly_step<kDppXor1, 1>(v);
    }
}

template <int M>
struct Pow2Ceil {
    static constexpr int v = M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : 16;
};

// ---- split-K ------------------------------------------------------------------
__device__ __forceinline__ void ws_store(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float ws_load(const float *p) {
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Called by every thread of the workgroup once this workgroup's partials of
// row block rb are stored (ws_store) and complete (s_waitcnt) in the waves that
// stored them.  The workgroup that draws the last ticket adds the split_k
// partials ws[rb][0..S)[m][rl] in split order and writes C.
__device__ __forceinline__ void splitk_complete(const KParams &p, int rb, unsigned *flag) {
    lds_barrier();
    if (threadIdx.x == 0) {
        const unsigned t = __hip_atomic_fetch_add(&p.tickets[rb], 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
        *flag = (t == (unsigned)(p.split_k - 1)) ? 1u : 0u;
    }
    lds_barrier();
    if (*flag) {
        const int NB = p.rows_per_wg;
        const int total = p.M * NB;
        const float *base = p.ws + (size_t)rb * p.split_k * total;
        for (int i = threadIdx.x; i < total; i += blockDim.x) {
            const int m = i / NB;
            const int rl = i - m * NB;
            const int row = rb * NB + rl;
            if (row < p.N) {
                float v = 0.0f;
                for (int s = 0; s < p.split_k; ++s) v += ws_load(base + (size_t)s * total + i);
                store_c(p, m, row, v);
            }
        }
        if (threadIdx.x == 0)
            __hip_atomic_store(&p.tickets[rb], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Work assignment of one workgroup.
struct WgPlan {
    int s;       // K slice
    int rb0;     // first row block
    int rbs;     // row-block stride
    int nblk;    // row blocks of this workgroup
    int wg_c0;   // first chunk of the slice
};

__device__ __forceinline__ WgPlan wg_plan(const KParams &p) {
    WgPlan w;
    const int S = p.split_k;
    w.rb0 = blockIdx.x / S;
    w.s = blockIdx.x - w.rb0 * S;
    w.rbs = gridDim.x / S;
    w.nblk = w.rb0 < p.num_rb ? (p.num_rb - w.rb0 + w.rbs - 1) / w.rbs : 0;
    w.wg_c0 = w.s * p.wg_chunks;
    return w;
}

// ---- VALU kernel --------------------------------------------------------------
// M: tokens (compile time); R: row slots per wave (4 rows each);
// PF: K-steps of B loads in flight (register ring depth).
template <int M, int R, int PF>
__global__ void __launch_bounds__(kMaxWaves * 64) skg_valu_kernel(KParams p) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    uint16_t *As = reinterpret_cast<uint16_t *>(smem);
    float *red = reinterpret_cast<float *>(smem + p.red_offset);
    unsigned *flag = reinterpret_cast<unsigned *>(smem + p.flag_offset);

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int l16 = lane & 15;
    const int slot = lane >> 4;
    const int wk = wave / p.waves_n;
    const int wn = wave - wk * p.waves_n;
    const WgPlan w = wg_plan(p);
    const int NB = p.rows_per_wg;
    const int SPB = p.wave_chunks / kValuStep;  // K steps per row block
    const int T = w.nblk * SPB;
    const int wv_c0 = w.wg_c0 + wk * p.wave_chunks;
    const int rl0 = wn * (4 * R) + slot;  // local row of slot r = 0

    // load cursor: row block lb, step lst
    int lb = 0, lst = 0;
    const uint16_t *rowp[R];
    auto set_rows = [&](int b) {
        const int rbase = (w.rb0 + b * w.rbs) * NB + rl0;
#pragma unroll
        for (int r = 0; r < R; ++r)
            rowp[r] = p.B + (int64_t)min(rbase + 4 * r, p.N - 1) * p.ldb;
    };
    auto issue = [&](uint4(&dst)[R]) {
        const int cb = wv_c0 + lst * kValuStep;
        const int c = cb + l16;
        if (cb + kValuStep <= p.nfull) {
#pragma unroll
            for (int r = 0; r < R; ++r) dst[r] = ldg16_stream(rowp[r] + (int64_t)c * kChunk);
        } else {
#pragma unroll
            for (int r = 0; r < R; ++r) dst[r] = load_chunk_masked<true>(rowp[r], c, p);
        }
        if (++lst == SPB) {
            lst = 0;
            if (++lb < w.nblk) set_rows(lb);
        }
    };

    uint4 buf[PF][R];
    if (w.nblk > 0) set_rows(0);
#pragma unroll
    for (int i = 0; i < PF; ++i)
        if (i < T) issue(buf[i]);

    stage_a(p, As, w.wg_c0);
    __syncthreads();

    float acc[R][M];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;

    constexpr int VP = Pow2Ceil<M>::v;
    const bool writer = l16 < M;
    const int m_out = l16;
    const uint16_t *ap = As + (wk * p.wave_chunks + l16) * kChunk;
    const int red_block = (p.waves_k - 1) * M * NB;  // floats per red buffer

    // epilogue of compute row block b: reduce, combine waves, write
    auto finish_block = [&](int b) {
        float res[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float v[VP];
#pragma unroll
            for (int j = 0; j < VP; ++j) v[j] = (j < M) ? acc[r][j] : 0.0f;
            reduce16<VP>(v, lane);
            res[r] = v[0];
        }
        const int rb = w.rb0 + b * w.rbs;
        if (p.waves_k > 1) {
            float *rbuf = red + (b & 1) * red_block;
            if (wk > 0 && writer)
#pragma unroll
                for (int r = 0; r < R; ++r)
                    rbuf[((wk - 1) * M + m_out) * NB + rl0 + 4 * r] = res[r];
            lds_barrier();
            if (wk == 0 && writer)
                for (int q = 1; q < p.waves_k; ++q)
#pragma unroll
                    for (int r = 0; r < R; ++r)
                        res[r] += rbuf[((q - 1) * M + m_out) * NB + rl0 + 4 * r];
        }
        const int row0 = rb * NB + rl0;
        if (p.split_k == 1) {
            if (wk == 0 && writer)
#pragma unroll
                for (int r = 0; r < R; ++r)
                    if (row0 + 4 * r < p.N) store_c(p, m_out, row0 + 4 * r, res[r]);
        } else if (p.two_pass) {
            if (wk == 0 && writer) {
                float *dst = p.ws + ((size_t)(rb * p.split_k + w.s) * M + m_out) * NB;
#pragma unroll
                for (int r = 0; r < R; ++r) dst[rl0 + 4 * r] = res[r];
            }
        } else {
            if (wk == 0) {
                if (writer) {
                    float *dst = p.ws + ((size_t)(rb * p.split_k + w.s) * M + m_out) * NB;
#pragma unroll
                    for (int r = 0; r < R; ++r) ws_store(dst + rl0 + 4 * r, res[r]);
                }
                __builtin_amdgcn_s_waitcnt(0);  // partial stores complete
            }
            splitk_complete(p, rb, flag);
        }
    };

    int cb = 0, cst = 0;  // compute cursor
    for (int t0 = 0; t0 < T; t0 += PF) {
#pragma unroll
        for (int i = 0; i < PF; ++i) {
            if (t0 + i < T) {
                const uint16_t *a_st = ap + cst * (kValuStep * kChunk);
                uint4 a[M];
#pragma unroll
                for (int m = 0; m < M; ++m) a[m] = lds16(a_st + m * p.lds_stride);
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int m = 0; m < M; ++m) acc[r][m] = dot8(a[m], buf[i][r], acc[r][m]);
                if (t0 + i + PF < T) issue(buf[i]);
                if (++cst == SPB) {
                    finish_block(cb);
#pragma unroll
                    for (int r = 0; r < R; ++r)
#pragma unroll
                        for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;
                    cst = 0;
                    ++cb;
                }
            }
        }
    }
}

// ---- MFMA kernel ------------------------------------------------------------
// Stage A[:, slice] in LDS in MFMA operand order: for each 32-wide K step, the
// 64 lane fragments (lane l: token m = l & 15, chunk l >> 4 of the step) lie
// contiguously, so the per-step operand read is one conflict-free 1 KB
// ds_read_b128.  One direct-to-LDS load per step block; tokens m >= M load
// row M-1 (the readers mask them to zero); chunks at or beyond K are written
// as (partial) zeros by ordinary LDS stores.
__device__ __forceinline__ void stage_a_frag(const KParams &p, uint16_t *As, int wg_c0) {
    const int lane = threadIdx.x & 63;
    const int nwaves = blockDim.x >> 6;
    const int m = min(lane & 15, p.M - 1);
    const uint16_t *rowp = p.A + (int64_t)m * p.lda;
    const int nblk = p.wg_chunks >> 2;  // 32-wide steps
    for (int blk = threadIdx.x >> 6; blk < nblk; blk += nwaves) {
        const int c = wg_c0 + 4 * blk + (lane >> 4);
        uint16_t *dst = As + blk * 64 * kChunk;
        if (c < p.nfull)
            lds_dma16(rowp + (int64_t)c * kChunk, dst);
        else
            sts16(dst + lane * kChunk, load_chunk_masked(rowp, c, p));
    }
}

// The MFMA B operand wants lane l to hold 8 consecutive k of row (l & 15);
// loading it that way makes every quarter-wave touch 16 rows (16 B each),
// which streams far slower than one 256-byte row segment per quarter-wave.
// So B is loaded with the VALU layout (lane l: row 4q + (l >> 4), chunk
// l & 15, q = 0..3 over four loads = 16 rows x 128 k) and transposed through
// a wave-private 4 KB LDS tile: (row r, chunk c) sits in 16-byte slot
// r * 16 + (c ^ r), so the writes (one row per quarter-wave) and the operand
// reads (16 rows, one chunk each per quarter-wave) both hit 16 distinct slots.
__device__ __forceinline__ int tile_slot(int r, int c) { return r * 16 + (c ^ r); }

// G: 16-row tiles per wave; PF: 128-wide K steps of loads in flight; AG: the
// activations of each step are loaded from global memory (L2-resident, in the
// same register ring as B, with the same row-segment layout) and transposed
// through their own wave-private tile, instead of being staged in LDS.
// M <= 16 at run time (activation rows m >= M are fed as zeros).
template <int G, int PF, bool AG>
__global__ void __launch_bounds__(kMaxWaves * 64) skg_mfma_kernel(KParams p) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    uint16_t *As = reinterpret_cast<uint16_t *>(smem);
    float *red = reinterpret_cast<float *>(smem + p.red_offset);
    unsigned *flag = reinterpret_cast<unsigned *>(smem + p.flag_offset);

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int lo = lane & 15;  // load: chunk within the step; operand: row / token
    const int hi = lane >> 4;  // load: row within a group of 4; operand: chunk of 4
    const int wk = wave / p.waves_n;
    const int wn = wave - wk * p.waves_n;
    const WgPlan w = wg_plan(p);
    const int NB = p.rows_per_wg;
    const int M = p.M;
    const int SPB = p.wave_chunks / kValuStep;
    const int T = w.nblk * SPB;
    const int wv_c0 = w.wg_c0 + wk * p.wave_chunks;
    const int rlw = wn * (16 * G);  // first local row of this wave
    constexpr int NT = G + (AG ? 1 : 0);  // transpose tiles per wave (B tiles, then A)
    uint4 *tile = reinterpret_cast<uint4 *>(smem + p.tr_offset) + wave * (NT * 256);
    // AG: activation rows 4q + hi of this lane (rows >= M read row M-1, masked)
    const int aq = (M + 3) >> 2;  // activation loads per step
    const uint16_t *arow[4];
    uint32_t amask[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        arow[q] = p.A + (int64_t)min(4 * q + hi, M - 1) * p.lda;
        amask[q] = (4 * q + hi < M) ? 0xFFFFFFFFu : 0u;
    }

    int lb = 0, lst = 0;
    const uint16_t *rowp[G][4];
    auto set_rows = [&](int b) {
        const int rbase = (w.rb0 + b * w.rbs) * NB + rlw + hi;
#pragma unroll
        for (int t = 0; t < G; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                rowp[t][q] = p.B + (int64_t)min(rbase + 16 * t + 4 * q, p.N - 1) * p.ldb;
    };
    auto issue = [&](uint4(&dst)[G][4], uint4(&adst)[4]) {
        const int cb = wv_c0 + lst * kValuStep;
        const int c = cb + lo;
        if (cb + kValuStep <= p.nfull) {
#pragma unroll
            for (int t = 0; t < G; ++t)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    dst[t][q] = ldg16_stream(rowp[t][q] + (int64_t)c * kChunk);
            if constexpr (AG)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (q < aq) adst[q] = ldg16(arow[q] + (int64_t)c * kChunk);
        } else {
#pragma unroll
            for (int t = 0; t < G; ++t)
#pragma unroll
                for (int q = 0; q < 4; ++q) dst[t][q] = load_chunk_masked<true>(rowp[t][q], c, p);
            if constexpr (AG)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (q < aq) adst[q] = load_chunk_masked(arow[q], c, p);
        }
        if (++lst == SPB) {
            lst = 0;
            if (++lb < w.nblk) set_rows(lb);
        }
    };

    uint4 buf[PF][G][4];
    uint4 abuf[PF][4];
    if (w.nblk > 0) set_rows(0);
#pragma unroll
    for (int i = 0; i < PF; ++i)
        if (i < T) issue(buf[i], abuf[i]);

    if constexpr (!AG) {
        stage_a_frag(p, As, w.wg_c0);
        __syncthreads();
    }

    f32x4_t acc[G];
#pragma unroll
    for (int t = 0; t < G; ++t) acc[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // LDS activation fragments of this wave: one 1 KB block per 32-wide step;
    // lanes of tokens m >= M zero what they read
    const uint16_t *ap = As + ((wk * p.wave_chunks) / 4 * 64 + lane) * kChunk;
    const uint32_t lane_mask = (lo < M) ? 0xFFFFFFFFu : 0u;
    const int red_block = (p.waves_k - 1) * M * NB;

    // acc[t][v] holds C[m = 4*hi + v][row = row block base + rlw + 16*t + lo]
    auto finish_block = [&](int b) {
        const int rb = w.rb0 + b * w.rbs;
        if (p.waves_k > 1) {
            float *rbuf = red + (b & 1) * red_block;
            if (wk > 0)
#pragma unroll
                for (int t = 0; t < G; ++t)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int m = 4 * hi + v;
                        if (m < M) rbuf[((wk - 1) * M + m) * NB + rlw + 16 * t + lo] = acc[t][v];
                    }
            lds_barrier();
            if (wk == 0)
                for (int q = 1; q < p.waves_k; ++q)
#pragma unroll
                    for (int t = 0; t < G; ++t)
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const int m = 4 * hi + v;
                            if (m < M) acc[t][v] += rbuf[((q - 1) * M + m) * NB + rlw + 16 * t + lo];
                        }
        }
        const int rowb = rb * NB + rlw + lo;
        if (p.split_k == 1) {
            if (wk == 0)
#pragma unroll
                for (int t = 0; t < G; ++t) {
                    const int row = rowb + 16 * t;
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int m = 4 * hi + v;
                        if (m < M && row < p.N) store_c(p, m, row, acc[t][v]);
                    }
                }
        } else if (p.two_pass) {
            if (wk == 0) {
                float *dst = p.ws + (size_t)(rb * p.split_k + w.s) * M * NB;
#pragma unroll
                for (int t = 0; t < G; ++t)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int m = 4 * hi + v;
                        if (m < M) dst[m * NB + rlw + 16 * t + lo] = acc[t][v];
                    }
            }
        } else {
            if (wk == 0) {
                float *dst = p.ws + (size_t)(rb * p.split_k + w.s) * M * NB;
#pragma unroll
                for (int t = 0; t < G; ++t)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int m = 4 * hi + v;
                        if (m < M) ws_store(dst + m * NB + rlw + 16 * t + lo, acc[t][v]);
                    }
                __builtin_amdgcn_s_waitcnt(0);  // partial stores complete
            }
            splitk_complete(p, rb, flag);
        }
    };

    int cb = 0, cst = 0;
    for (int t0 = 0; t0 < T; t0 += PF) {
#pragma unroll
        for (int i = 0; i < PF; ++i) {
            if (t0 + i < T) {
                // transpose this step's B (and A) through the wave's LDS tiles
#pragma unroll
                for (int t = 0; t < G; ++t)
#pragma unroll
                    for (int q = 0; q < 4; ++q) tile[t * 256 + tile_slot(4 * q + hi, lo)] = buf[i][t][q];
                if constexpr (AG) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        uint4 v = make_uint4(0u, 0u, 0u, 0u);
                        if (q < aq) {
                            v = abuf[i][q];
                            v.x &= amask[q];
                            v.y &= amask[q];
                            v.z &= amask[q];
                            v.w &= amask[q];
                        }
                        tile[G * 256 + tile_slot(4 * q + hi, lo)] = v;
                    }
                }
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    uint4 a;
                    if constexpr (AG) {
                        a = tile[G * 256 + tile_slot(lo, 4 * s + hi)];
                    } else {
                        a = lds16(ap + (cst * 4 + s) * (64 * kChunk));
                        a.x &= lane_mask;
                        a.y &= lane_mask;
                        a.z &= lane_mask;
                        a.w &= lane_mask;
                    }
                    const bf16x8_t av = __builtin_bit_cast(bf16x8_t, a);
#pragma unroll
                    for (int t = 0; t < G; ++t) {
                        const uint4 bv = tile[t * 256 + tile_slot(lo, 4 * s + hi)];
                        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            av, __builtin_bit_cast(bf16x8_t, bv), acc[t], 0, 0, 0);
                    }
                }
                if (t0 + i + PF < T) issue(buf[i], abuf[i]);
                if (++cst == SPB) {
                    finish_block(cb);
#pragma unroll
                    for (int t = 0; t < G; ++t) acc[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
                    cst = 0;
                    ++cb;
                }
            }
        }
    }
}

// Instantiation list for one M, in the order of kValuVariants.
#define SKG_VALU_ROW(M)                                                           \
    {skg_valu_kernel<M, 1, 4>, skg_valu_kernel<M, 1, 8>, skg_valu_kernel<M, 2, 2>, \
     skg_valu_kernel<M, 2, 4>, skg_valu_kernel<M, 4, 2>, skg_valu_kernel<M, 4, 4>}

}  // namespace
}  // namespace skg

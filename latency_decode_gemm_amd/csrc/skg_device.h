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
//  * One launch streams B exactly once.  A workgroup owns a block of rows of
//    B (rows_per_wg) and one slice of K; its waves split the rows (waves_n)
//    and the slice (waves_k).  A[:, slice] is staged once per workgroup in
//    LDS (zero beyond K) and re-read from LDS; B goes HBM -> VGPRs directly.
//  * VALU inner product: 16 lanes per row of B, so one 64-lane dwordx4 load
//    covers 4 rows x 256 contiguous bytes; each lane keeps `depth` K-steps of
//    loads in flight in a register ring and multiplies with v_dot2c_f32_bf16
//    (two bf16 products added into fp32).  At the end the 16 lanes of a row
//    are combined with a DPP reduce-scatter (row_mirror, row_half_mirror,
//    quad_perm), which leaves lane i of the row group with the sum for m = i.
//  * MFMA inner product (v_mfma_f32_16x16x32_bf16): the activations are the
//    16-row operand (rows m >= M are zero), 16 rows of B are the 16 columns;
//    the instruction performs the K reduction, so no cross-lane step remains.
//  * Cross-wave (waves_k > 1): partials go through LDS and wave 0 adds them
//    in wave order.  Cross-workgroup (split_k > 1): each workgroup writes its
//    fp32 partial tile, releases it at agent scope and takes a ticket; the
//    workgroup that draws the last ticket acquires, sums the split_k partials
//    in split order and writes C, then resets the ticket.  Nothing waits for
//    another workgroup, and the summation order never depends on timing, so
//    results are bit-reproducible.
//  * Epilogue: fp32 stores, or bf16 round-to-nearest-even, at C[m*ldc + n];
//    other bytes of C are never written.
#pragma once

#include "skg_internal.h"

namespace skg {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ldg16(const uint16_t *p) {
    return *reinterpret_cast<const uint4 *>(p);
}

__device__ __forceinline__ uint4 lds16(const uint16_t *p) {
    return *reinterpret_cast<const uint4 *>(p);
}

__device__ __forceinline__ void sts16(uint16_t *p, uint4 v) {
    *reinterpret_cast<uint4 *>(p) = v;
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

// One 8-element chunk of row `row` starting at k = 8*c, with everything at
// k >= K (and every chunk outside [0, c_end)) read as zero.
__device__ __forceinline__ uint4 load_chunk_masked(const uint16_t *rowp, int c, int c_end,
                                                   const KParams &p) {
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (c < c_end) {
        if (c < p.nfull) {
            v = ldg16(rowp + (int64_t)c * kChunk);
        } else {
            // the one chunk that straddles K (K % 8 != 0)
            uint32_t w[4] = {0u, 0u, 0u, 0u};
            const int k0 = c * kChunk;
#pragma unroll
            for (int e = 0; e < kChunk; ++e) {
                if (k0 + e < p.K) {
                    uint32_t h = rowp[k0 + e];
                    w[e >> 1] |= h << (16 * (e & 1));
                }
            }
            v = make_uint4(w[0], w[1], w[2], w[3]);
        }
    }
    return v;
}

// Stage A[m, 8*wg_c0 : 8*(wg_c0 + wg_chunks)) for m < M into LDS rows of
// p.lds_stride elements; zeros beyond K.  Up to 8 rows' loads are issued
// before their LDS stores so the latencies overlap.
template <int MT>  // MT: compile-time upper bound of M
__device__ __forceinline__ void stage_a(const KParams &p, uint16_t *As, int wg_c0) {
    const int nch = p.wg_chunks;
    for (int cc = threadIdx.x; cc < nch; cc += blockDim.x) {
        const int c = wg_c0 + cc;
#pragma unroll
        for (int m0 = 0; m0 < MT; m0 += 8) {
            uint4 v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int m = m0 + i;
                if (m < MT && m < p.M) v[i] = load_chunk_masked(p.A + (int64_t)m * p.lda, c, p.nck, p);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int m = m0 + i;
                if (m < MT && m < p.M) sts16(As + m * p.lds_stride + cc * kChunk, v[i]);
            }
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

// ---- split-K completion -----------------------------------------------------
// Called by every thread of the workgroup after it has stored its partials
// ws[((rb*S + s)*M + m)*NB + rl].  The workgroup that draws the last ticket
// adds the S partials of the row block in split order and writes C.
__device__ __forceinline__ void splitk_complete(const KParams &p, int rb, unsigned *flag) {
    __threadfence();  // release this thread's partial stores at agent scope
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned t = __hip_atomic_fetch_add(&p.tickets[rb], 1u, __ATOMIC_ACQ_REL,
                                                  __HIP_MEMORY_SCOPE_AGENT);
        *flag = (t == (unsigned)(p.split_k - 1)) ? 1u : 0u;
    }
    __syncthreads();
    if (*flag) {
        __threadfence();  // acquire: the other workgroups' partials are visible
        const int NB = p.rows_per_wg;
        const int total = p.M * NB;
        const float *base = p.ws + (size_t)rb * p.split_k * total;
        for (int i = threadIdx.x; i < total; i += blockDim.x) {
            const int m = i / NB;
            const int rl = i - m * NB;
            const int row = rb * NB + rl;
            if (row < p.N) {
                float v = 0.0f;
                for (int s = 0; s < p.split_k; ++s) v += base[(size_t)s * total + i];
                store_c(p, m, row, v);
            }
        }
        if (threadIdx.x == 0)
            __hip_atomic_store(&p.tickets[rb], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Per-workgroup K range and per-wave K part, in chunks.
struct KRange {
    int wg_c0, wv_c0, wv_c1, nsteps, tail_c0;
    bool has_tail;
};

__device__ __forceinline__ KRange k_range(const KParams &p, int s, int wk, int step) {
    KRange r;
    r.wg_c0 = s * p.wg_chunks;
    const int wg_c1 = min(r.wg_c0 + p.wg_chunks, p.nck);
    r.wv_c0 = r.wg_c0 + wk * p.wave_chunks;
    r.wv_c1 = min(r.wv_c0 + p.wave_chunks, wg_c1);
    const int fc1 = min(r.wv_c1, p.nfull);
    r.nsteps = fc1 > r.wv_c0 ? (fc1 - r.wv_c0) / step : 0;
    r.tail_c0 = r.wv_c0 + r.nsteps * step;
    r.has_tail = r.tail_c0 < r.wv_c1;
    return r;
}

// ---- VALU kernel --------------------------------------------------------------
// M: tokens (compile time); R: row slots per wave (4 rows each);
// PF: K-steps of B loads in flight (register ring depth).
template <int M, int R, int PF>
__global__ void __launch_bounds__(kMaxWaves * 64) skg_valu_kernel(KParams p) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    uint16_t *As = reinterpret_cast<uint16_t *>(smem);
    float *red = reinterpret_cast<float *>(smem + p.red_offset);
    unsigned *flag = reinterpret_cast<unsigned *>(smem + p.red_offset) +
                     (p.waves_k - 1) * M * p.rows_per_wg;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int l16 = lane & 15;
    const int slot = lane >> 4;
    const int wk = wave / p.waves_n;
    const int wn = wave - wk * p.waves_n;
    const int rb = blockIdx.x / p.split_k;
    const int s = blockIdx.x - rb * p.split_k;

    const KRange kr = k_range(p, s, wk, kValuStep);
    const int rl0 = wn * (4 * R) + slot;  // local row of slot r = 0
    const int row0 = rb * p.rows_per_wg + rl0;

    const uint16_t *bp[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int row = min(row0 + 4 * r, p.N - 1);
        bp[r] = p.B + (int64_t)row * p.ldb + (int64_t)(kr.wv_c0 + l16) * kChunk;
    }

    uint4 buf[PF][R];
#pragma unroll
    for (int i = 0; i < PF; ++i)
        if (i < kr.nsteps)
#pragma unroll
            for (int r = 0; r < R; ++r) buf[i][r] = ldg16(bp[r] + i * (kValuStep * kChunk));

    stage_a<M>(p, As, kr.wg_c0);
    __syncthreads();

    float acc[R][M];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;

    const uint16_t *ap = As + (kr.wv_c0 - kr.wg_c0 + l16) * kChunk;
    for (int st = 0; st < kr.nsteps; st += PF) {
#pragma unroll
        for (int i = 0; i < PF; ++i) {
            if (st + i < kr.nsteps) {
                uint4 a[M];
#pragma unroll
                for (int m = 0; m < M; ++m)
                    a[m] = lds16(ap + m * p.lds_stride + (st + i) * (kValuStep * kChunk));
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int m = 0; m < M; ++m) acc[r][m] = dot8(a[m], buf[i][r], acc[r][m]);
                if (st + i + PF < kr.nsteps)
#pragma unroll
                    for (int r = 0; r < R; ++r)
                        buf[i][r] = ldg16(bp[r] + (st + i + PF) * (kValuStep * kChunk));
            }
        }
    }
    if (kr.has_tail) {
        const int c = kr.tail_c0 + l16;
        uint4 b[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = min(row0 + 4 * r, p.N - 1);
            b[r] = load_chunk_masked(p.B + (int64_t)row * p.ldb, c, kr.wv_c1, p);
        }
        const uint16_t *apt = As + (c - kr.wg_c0) * kChunk;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const uint4 a = lds16(apt + m * p.lds_stride);
#pragma unroll
            for (int r = 0; r < R; ++r) acc[r][m] = dot8(a, b[r], acc[r][m]);
        }
    }

    // 16 lanes of a row -> lane l16 holds the sum for m = l16 (if l16 < M)
    constexpr int VP = Pow2Ceil<M>::v;
    float res[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        float v[VP];
#pragma unroll
        for (int j = 0; j < VP; ++j) v[j] = (j < M) ? acc[r][j] : 0.0f;
        reduce16<VP>(v, lane);
        res[r] = v[0];
    }
    const bool writer = l16 < M;
    const int m = l16;
    const int NB = p.rows_per_wg;

    if (p.waves_k > 1) {
        if (wk > 0 && writer)
#pragma unroll
            for (int r = 0; r < R; ++r) red[((wk - 1) * M + m) * NB + rl0 + 4 * r] = res[r];
        __syncthreads();
        if (wk == 0 && writer)
            for (int w = 1; w < p.waves_k; ++w)
#pragma unroll
                for (int r = 0; r < R; ++r) res[r] += red[((w - 1) * M + m) * NB + rl0 + 4 * r];
    }

    if (p.split_k == 1) {
        if (wk == 0 && writer)
#pragma unroll
            for (int r = 0; r < R; ++r)
                if (row0 + 4 * r < p.N) store_c(p, m, row0 + 4 * r, res[r]);
    } else {
        if (wk == 0 && writer) {
            float *dst = p.ws + ((size_t)(rb * p.split_k + s) * M + m) * NB;
#pragma unroll
            for (int r = 0; r < R; ++r) dst[rl0 + 4 * r] = res[r];
        }
        splitk_complete(p, rb, flag);
    }
}

// ---- MFMA kernel ------------------------------------------------------------
// G: 16-row tiles per wave; PF: K-steps of B loads in flight.  M <= 16 at run
// time (activation rows m >= M are fed as zeros).
template <int G, int PF>
__global__ void __launch_bounds__(kMaxWaves * 64) skg_mfma_kernel(KParams p) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    uint16_t *As = reinterpret_cast<uint16_t *>(smem);
    float *red = reinterpret_cast<float *>(smem + p.red_offset);
    unsigned *flag = reinterpret_cast<unsigned *>(smem + p.red_offset) +
                     (p.waves_k - 1) * p.M * p.rows_per_wg;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int j = lane & 15;   // operand row: token m for A, row of B for B
    const int g4 = lane >> 4;  // which 8-element chunk of the 32-wide K step
    const int wk = wave / p.waves_n;
    const int wn = wave - wk * p.waves_n;
    const int rb = blockIdx.x / p.split_k;
    const int s = blockIdx.x - rb * p.split_k;

    const KRange kr = k_range(p, s, wk, kMfmaStep);
    const int rlw = wn * (16 * G);           // first local row of this wave
    const int rowb = rb * p.rows_per_wg + rlw;  // first global row of this wave

    const uint16_t *bp[G];
#pragma unroll
    for (int t = 0; t < G; ++t) {
        const int row = min(rowb + 16 * t + j, p.N - 1);
        bp[t] = p.B + (int64_t)row * p.ldb + (int64_t)(kr.wv_c0 + g4) * kChunk;
    }

    uint4 buf[PF][G];
#pragma unroll
    for (int i = 0; i < PF; ++i)
        if (i < kr.nsteps)
#pragma unroll
            for (int t = 0; t < G; ++t) buf[i][t] = ldg16(bp[t] + i * (kMfmaStep * kChunk));

    stage_a<16>(p, As, kr.wg_c0);
    __syncthreads();

    f32x4_t acc[G];
#pragma unroll
    for (int t = 0; t < G; ++t) acc[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // rows m >= M of the activation operand are zero: read a valid row and mask
    const uint32_t amask = (j < p.M) ? 0xFFFFFFFFu : 0u;
    const int jm = min(j, p.M - 1);
    const uint16_t *ap = As + jm * p.lds_stride + (kr.wv_c0 - kr.wg_c0 + g4) * kChunk;

    for (int st = 0; st < kr.nsteps; st += PF) {
#pragma unroll
        for (int i = 0; i < PF; ++i) {
            if (st + i < kr.nsteps) {
                uint4 a = lds16(ap + (st + i) * (kMfmaStep * kChunk));
                a.x &= amask; a.y &= amask; a.z &= amask; a.w &= amask;
                const bf16x8_t av = __builtin_bit_cast(bf16x8_t, a);
#pragma unroll
                for (int t = 0; t < G; ++t)
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        av, __builtin_bit_cast(bf16x8_t, buf[i][t]), acc[t], 0, 0, 0);
                if (st + i + PF < kr.nsteps)
#pragma unroll
                    for (int t = 0; t < G; ++t)
                        buf[i][t] = ldg16(bp[t] + (st + i + PF) * (kMfmaStep * kChunk));
            }
        }
    }
    if (kr.has_tail) {
        const int c = kr.tail_c0 + g4;
        uint4 a = lds16(As + jm * p.lds_stride + (c - kr.wg_c0) * kChunk);
        a.x &= amask; a.y &= amask; a.z &= amask; a.w &= amask;
        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, a);
#pragma unroll
        for (int t = 0; t < G; ++t) {
            const int row = min(rowb + 16 * t + j, p.N - 1);
            const uint4 b = load_chunk_masked(p.B + (int64_t)row * p.ldb, c, kr.wv_c1, p);
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, b),
                                                             acc[t], 0, 0, 0);
        }
    }

    // acc[t][v] holds C[m = 4*g4 + v][row = rowb + 16*t + j]
    const int NB = p.rows_per_wg;
    const int M = p.M;
    if (p.waves_k > 1) {
        if (wk > 0)
#pragma unroll
            for (int t = 0; t < G; ++t)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int m = 4 * g4 + v;
                    if (m < M) red[((wk - 1) * M + m) * NB + rlw + 16 * t + j] = acc[t][v];
                }
        __syncthreads();
        if (wk == 0)
            for (int w = 1; w < p.waves_k; ++w)
#pragma unroll
                for (int t = 0; t < G; ++t)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int m = 4 * g4 + v;
                        if (m < M) acc[t][v] += red[((w - 1) * M + m) * NB + rlw + 16 * t + j];
                    }
    }

    if (p.split_k == 1) {
        if (wk == 0)
#pragma unroll
            for (int t = 0; t < G; ++t) {
                const int row = rowb + 16 * t + j;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int m = 4 * g4 + v;
                    if (m < M && row < p.N) store_c(p, m, row, acc[t][v]);
                }
            }
    } else {
        if (wk == 0) {
            float *dst = p.ws + (size_t)(rb * p.split_k + s) * M * NB;
#pragma unroll
            for (int t = 0; t < G; ++t)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int m = 4 * g4 + v;
                    if (m < M) dst[m * NB + rlw + 16 * t + j] = acc[t][v];
                }
        }
        splitk_complete(p, rb, flag);
    }
}

// Instantiation list for one M, in the order of kValuVariants.
#define SKG_VALU_ROW(M)                                                           \
    {skg_valu_kernel<M, 1, 4>, skg_valu_kernel<M, 1, 8>, skg_valu_kernel<M, 2, 2>, \
     skg_valu_kernel<M, 2, 4>, skg_valu_kernel<M, 4, 2>, skg_valu_kernel<M, 4, 4>}

}  // namespace
}  // namespace skg

// skg_device.h -- gfx950 kernels for C[M,N] = A[M,K] . B[N,K]^T, M <= 16 (the
// matrix-core kernels: M <= 64 with up to four token tiles of 16).
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
//    of rows_per_wg rows (or dealt evenly, one block per workgroup); K is cut
//    into split_k slices.  A workgroup owns one K slice and a strided set of
//    row blocks (blockIdx / split_k, then every gridDim / split_k-th), so it
//    stages A[:, slice] in LDS once (zero beyond K) and then streams all of
//    its row blocks.  Its waves split the rows of a block (waves_n) and the
//    slice (waves_k, equal parts).
//  * Every wave runs one flat stream of K steps over all its row blocks, with
//    `depth` steps of B loads in flight in a register ring (or, in the
//    LDS-ring MFMA kernel, in LDS tiles filled by direct global-to-LDS
//    loads); the loads of the next row block are already in flight while the
//    current block is reduced and written.  Barriers inside that stream wait
//    for LDS traffic only, so they never drain the ring.
//  * VALU inner product: 16 lanes per row of B, so one 64-lane dwordx4 load
//    covers 4 rows x 256 contiguous bytes; products by v_dot2c_f32_bf16 (two
//    bf16 products added into fp32).  The 16 lanes of a row are combined with
//    a DPP reduce-scatter (row_mirror, row_half_mirror, quad_perm) that leaves
//    lane i of the row group with the sum for token m = i.
//  * MFMA inner product (v_mfma_f32_16x16x32_bf16): the activations are the
//    16-row operand (rows m >= M are never stored), 16 rows of B are the 16
//    columns; the instruction performs the K reduction, so no cross-lane step
//    remains.
//  * Cross-wave (waves_k > 1): partials go through LDS (double-buffered per
//    row block) and wave 0 adds them in wave order.  Cross-workgroup
//    (split_k > 1, one pass): the split_k partials of each output are
//    combined pairwise along a fixed binary tree, the value itself carried by
//    a 64-bit atomic exchange on the tree node's slot; whichever workgroup
//    arrives second at a node adds left + right and climbs, and the one that
//    completes the root writes C.  Nothing waits for another workgroup, and
//    the summation order is the tree's whatever the arrival order, so results
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

// The same as an instruction the compiler does not see into: its wait
// insertion would otherwise drain every load before any LDS read that may
// alias such a write (so a ring of them would never have more than one step
// in flight).  The caller waits for the data itself (wait_vmcnt).  lds_addr
// is the wave-uniform LDS byte address of lane 0's 16 bytes; NT marks the
// load non-temporal (weights, read once).  m0 is set inside the statement
// (one wait state before the load reads it); in the kernels that use this,
// no compiler-generated instruction reads m0.
__device__ __forceinline__ uint32_t lds_addr_of(const void *lds_ptr) {
    typedef __attribute__((address_space(3))) const void *lptr_t;
    return __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(lptr_t)(lds_ptr));
}
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 in the clobber list
template <bool NT>
__device__ __forceinline__ void lds_dma16_raw(const uint16_t *gsrc, uint32_t lds_addr) {
    if constexpr (NT)
        __asm__ volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
                         :
                         : "v"(gsrc), "s"(lds_addr)
                         : "memory", "m0");
    else
        __asm__ volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                         :
                         : "v"(gsrc), "s"(lds_addr)
                         : "memory", "m0");
}
#pragma clang diagnostic pop

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

// Eight bf16 activations times eight fp32 weights (w0: elements 0..3, w1:
// 4..7), one fused multiply-add each, in element order.  The bf16 -> fp32
// widening is exact (the 16 bits become the upper half of the fp32 word).
__device__ __forceinline__ float bf_lo(uint32_t x) { return __builtin_bit_cast(float, x << 16); }
__device__ __forceinline__ float bf_hi(uint32_t x) {
    return __builtin_bit_cast(float, x & 0xFFFF0000u);
}
__device__ __forceinline__ float u2f(uint32_t x) { return __builtin_bit_cast(float, x); }
__device__ __forceinline__ float dot8_f32w(const uint4 &a, const uint4 &w0, const uint4 &w1,
                                           float c) {
    c = __builtin_fmaf(bf_lo(a.x), u2f(w0.x), c);
    c = __builtin_fmaf(bf_hi(a.x), u2f(w0.y), c);
    c = __builtin_fmaf(bf_lo(a.y), u2f(w0.z), c);
    c = __builtin_fmaf(bf_hi(a.y), u2f(w0.w), c);
    c = __builtin_fmaf(bf_lo(a.z), u2f(w1.x), c);
    c = __builtin_fmaf(bf_hi(a.z), u2f(w1.y), c);
    c = __builtin_fmaf(bf_lo(a.w), u2f(w1.z), c);
    c = __builtin_fmaf(bf_hi(a.w), u2f(w1.w), c);
    return c;
}

// fp32 -> bf16, round to nearest even; NaN stays a (quiet) NaN.
// (both results formed and one selected: no branch per value in the
// epilogues, where one wave per SIMD runs them back to back)
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    const uint32_t u = __builtin_bit_cast(uint32_t, f);
    const uint32_t rounded = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    const uint32_t quiet_nan = (u >> 16) | 0x0040u;
    return (uint16_t)(((u & 0x7FFFFFFFu) > 0x7F800000u) ? quiet_nan : rounded);
}

__device__ __forceinline__ void store_c(const KParams &p, int m, int n, float v) {
    const int64_t off = (int64_t)m * p.ldc + n;
    if (p.out_bf16)
        reinterpret_cast<uint16_t *>(p.C)[off] = f32_to_bf16_rne(v);
    else
        reinterpret_cast<float *>(p.C)[off] = v;
}

// The outputs of one accumulator fragment lane: tokens m0 .. m0 + 3 (those
// below M) of column n, the output type tested once and the rows of C
// reached by adding ldc.
__device__ __forceinline__ void store_c4(const KParams &p, int m0, int n, const f32x4_t &v) {
    const int64_t ld = p.ldc;
    const int64_t off = (int64_t)m0 * ld + n;
    if (p.out_bf16) {
        uint16_t *c = reinterpret_cast<uint16_t *>(p.C) + off;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (m0 + j < p.M) c[j * ld] = f32_to_bf16_rne(v[j]);
    } else {
        float *c = reinterpret_cast<float *>(p.C) + off;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (m0 + j < p.M) c[j * ld] = v[j];
    }
}

// ---- K tail ------------------------------------------------------------------
// Every load is one 16-byte window.  Chunk c < nfull is read in place.  The
// chunk that straddles K (K % 8 != 0) is read as the window ending exactly at
// K, and chunks beyond K re-read that same window, so no load ever leaves
// [0, K) of its row (K >= 8; smaller K has a kernel of its own).  The mask
// below then keeps only what belongs to chunk c: all of it for c < nfull,
// the last K % 8 elements for the straddling chunk, nothing beyond K.  Both
// operands are masked, so padding (even NaN) never meets a product.
__device__ __forceinline__ int64_t window_off(int c, const KParams &p) {
    return (int64_t)min(c * kChunk, p.K - kChunk);
}

// First window position that belongs to chunk c (0 inside K, 8 beyond it).
__device__ __forceinline__ int tail_j0(int c, const KParams &p) {
    return (c < p.nfull) ? 0 : (c < p.nck ? kChunk - (p.K - p.nfull * kChunk) : kChunk);
}

__device__ __forceinline__ uint4 tail_mask(int c, const KParams &p) {
    const int j0 = tail_j0(c, p);
    uint32_t w[4];
#pragma unroll
    for (int d = 0; d < 4; ++d)
        w[d] = ((2 * d >= j0) ? 0x0000FFFFu : 0u) | ((2 * d + 1 >= j0) ? 0xFFFF0000u : 0u);
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// The same mask for half h (window positions 4h .. 4h + 3) of a window of
// eight fp32 weights.
__device__ __forceinline__ uint4 tail_mask_f32(int c, const KParams &p, int h) {
    const int j0 = tail_j0(c, p);
    uint32_t w[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) w[d] = (4 * h + d >= j0) ? 0xFFFFFFFFu : 0u;
    return make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ __forceinline__ uint4 and4(uint4 v, uint4 m) {
    return make_uint4(v.x & m.x, v.y & m.y, v.z & m.z, v.w & m.w);
}

// Chunk c of the row at rowp as the kernels see it (window + mask).
__device__ __forceinline__ uint4 load_chunk_tail(const uint16_t *rowp, int c, const KParams &p) {
    return and4(ldg16(rowp + window_off(c, p)), tail_mask(c, p));
}

// Stage A[m, 8*wg_c0 : 8*(wg_c0 + wg_chunks)) for m < M into LDS rows of
// p.lds_stride elements.  Each wave moves blocks of 64 chunks (1 KB, one row)
// straight into LDS; chunks from nfull on are written by ordinary LDS stores
// in the tail form above.  The caller's barrier waits for all of it.
__device__ __forceinline__ void stage_a(const KParams &p, uint16_t *As, int wg_c0) {
    const int lane = threadIdx.x & 63;
    const int nwaves = p.waves_n * p.waves_k;
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
                sts16(dst + lane * kChunk, load_chunk_tail(rowp, c, p));
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
// Slot word of a tree node: the fp32 bits of a partial sum in the upper half,
// the side it came from (0 left, 1 right) in bit 1, and bit 0 set, so an
// empty slot (0) differs from every partial, -0.0 and NaN included.
__device__ __forceinline__ unsigned long long slot_word(float v, int side) {
    return ((unsigned long long)__builtin_bit_cast(uint32_t, v) << 32) |
           ((unsigned long long)side << 1) | 1ull;
}

// Rows of row block rb: [start, start + count).  Uniform blocks of
// rows_per_wg rows (the last one cut at N), or, with SKG_BACKEND_EVEN, the N
// rows dealt evenly over num_rb blocks.  Loads clamp a local row to
// count - 1; stores take local rows < count only.
__device__ __forceinline__ void block_rows(const KParams &p, int rb, int &start, int &count) {
    if (p.even) {
        // rb N / num_rb = rb q + rb r / num_rb with N = q num_rb + r; rb r <
        // num_rb^2 <= 2^28, so 32-bit unsigned arithmetic is exact
        const unsigned nrb = (unsigned)p.num_rb, r = (unsigned)p.even_r;
        start = rb * p.even_q + (int)(((unsigned)rb * r) / nrb);
        count = p.even_q + (int)(((unsigned)(rb + 1) * r) / nrb - ((unsigned)rb * r) / nrb);
    } else {
        start = rb * p.rows_per_wg;
        count = min(p.rows_per_wg, p.N - start);
    }
}

// Combines this workgroup's partial v of output (m, local row rl) of row block
// rb, K slice sidx, with the other slices' partials.  The split_k slices are
// the leaves of a binary tree: at each level, entries 2j and 2j + 1 meet at
// node j (an odd last entry passes up unchanged), and the node's slot
// (p.slots, [row block][node][m][local row], zero between calls) takes
// exactly two exchanges per call.  The first to exchange finds the slot
// empty and stops; the second finds its sibling's partial, forms left + right
// (a fixed order, whichever arrived first), empties the slot for the next
// call and carries the sum one level up.  Returns true in the thread that
// completes the root, with the full sum in v.  The partials travel inside the
// atomic operations on one location each: the second exchange reads the first
// by the atomicity of read-modify-write, so no fence and no other memory is
// involved (relaxed, agent scope).  Slot indices fit 31 bits (the
// configuration check rejects more slots), so they are formed in 32-bit
// arithmetic.
__device__ __forceinline__ bool splitk_combine(const KParams &p, int rb, int sidx, int m, int rl,
                                               float &v) {
    const int S = p.split_k;
    int idx = sidx, width = S, node0 = 0;  // node0: first node of this level
    while (width > 1) {
        const int pairs = width >> 1;
        if (idx < 2 * pairs) {
            const int side = idx & 1;
            const unsigned si =
                (((unsigned)rb * (S - 1) + node0 + (idx >> 1)) * p.M + m) * p.rows_per_wg + rl;
            unsigned long long *slot = p.slots + si;
            const unsigned long long old = __hip_atomic_exchange(
                slot, slot_word(v, side), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (old == 0ull) return false;
            const float other = __builtin_bit_cast(float, (uint32_t)(old >> 32));
            v = side ? other + v : v + other;
            __hip_atomic_store(slot, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        node0 += pairs;
        idx >>= 1;
        width = (width + 1) >> 1;
    }
    return true;
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
    w.rbs = p.grid_rb;
    w.nblk = w.rb0 < p.num_rb ? (p.num_rb - w.rb0 + w.rbs - 1) / w.rbs : 0;
    w.wg_c0 = w.s * p.wg_chunks;
    return w;
}

// ---- epilogue ------------------------------------------------------------------
// A row block whose K range is covered by one wave is written straight from
// that wave's registers.  Otherwise (waves_k > 1, or the single-pass split-K
// backend, which combines per output) each wave parks its partial sums of
// each row block in LDS (the stash), and after the stream the workgroup's
// threads add the waves_k partials of an output in wave order and write C
// (split_k == 1), the split's partial (two-pass), or combine it with the other
// slices' (splitk_combine; the thread that completes the sum writes C).
__device__ __forceinline__ bool direct_write(const KParams &p) {
    return p.waves_k == 1 && (p.split_k == 1 || p.two_pass);
}

// The workgroup's K-wave sum v of output (token m, local row rl) of row block
// rb (rows [bst, bst + bcnt)).
__device__ __forceinline__ void finish_output(const KParams &p, const WgPlan &w, int rb, int bst,
                                              int bcnt, int m, int rl, float v) {
    if (p.split_k == 1) {
        if (rl < bcnt) store_c(p, m, bst + rl, v);
    } else if (p.two_pass) {
        p.ws[((size_t)(rb * p.split_k + w.s) * p.M + m) * p.rows_per_wg + rl] = v;
    } else if (rl < bcnt) {
        if (splitk_combine(p, rb, w.s, m, rl, v)) store_c(p, m, bst + rl, v);
    }
}

// VALU kernels (R row slots of 4 rows per wave): the stash is [row block]
// [K-wave][m][local row].  The thread of K-wave wk, N-wave wn and lane l takes
// local row 4 R wn + (l mod 4 R) and tokens l / (4 R) + (16 / R)(wk + waves_k
// i): each output once, consecutive lanes on consecutive rows (conflict-free
// stash reads, coalesced stores), and no division (the waves of a SIMD run
// the epilogue alone after the stream, where a chain of per-thread divisions
// cost half a microsecond).  The waves_k partials are added in K-wave order.
// bst0 and bcnt0: the rows of the workgroup's first row block.
template <int R>
__device__ __forceinline__ void write_blocks(const KParams &p, const WgPlan &w, const float *stash,
                                             int bst0, int bcnt0, int wk, int wn, int lane) {
    __syncthreads();
    const int NB = p.rows_per_wg;  // 4 R waves_n
    const int M = p.M;
    const int rl = 4 * R * wn + (lane & (4 * R - 1));
    const int mstep = (16 / R) * p.waves_k;
    for (int b = 0; b < w.nblk; ++b) {
        const int rb = w.rb0 + b * w.rbs;
        int bst = bst0, bcnt = bcnt0;
        if (b > 0) block_rows(p, rb, bst, bcnt);
        const float *blk = stash + b * p.waves_k * M * NB + rl;
        for (int m = lane / (4 * R) + (16 / R) * wk; m < M; m += mstep) {
            float v = blk[m * NB];
            for (int q = 1; q < p.waves_k; ++q) v += blk[(q * M + m) * NB];
            finish_output(p, w, rb, bst, bcnt, m, rl, v);
        }
    }
}

// Matrix-core kernels: each wave parks its accumulators in their fragment
// layout, f32x4 number (((b waves_k + q) waves_n + wq) G + t) MT + mt) 64 +
// lane for row block b, K-wave q, N-wave wq, row tile t and token tile mt;
// lane 16 hi + lo holds tokens 16 mt + 4 hi + j (j = 0..3) of local row
// 16 G wq + 16 t + lo.  Threads take whole fragments, wave r taking fragments
// r, r + (its waves), ... at its own lane: every stash read is one 16-byte
// read by consecutive lanes (no bank conflicts), the waves_k partials added
// element by element in wave order, and the index work is per lane and
// fragment (the waves of a SIMD run it alone after the stream, so a chain of
// per-thread divisions there cost half a microsecond).  Under the single-pass
// split with more threads than fragments, each thread takes single outputs
// instead, so that the outputs' chains of exchanges run side by side: the
// thread of K-wave wk, N-wave wn and lane l takes local rows 16 G wn + 16 t +
// (l & 15) (t < G) and tokens (l >> 4) + 4 (wk + waves_k i) (each output once,
// found without divisions); those stash reads meet two to a bank, and there
// are few per thread.  bst0 and bcnt0: the rows of the workgroup's first row
// block, computed before.
template <int G, int MT>
__device__ __forceinline__ void write_blocks_frag(const KParams &p, const WgPlan &w,
                                                  const f32x4_t *stash, int bst0, int bcnt0,
                                                  int wk, int wn, int lane) {
    __syncthreads();
    const int nthr = 64 * p.waves_n * p.waves_k;
    const int per_q = p.waves_n * G * MT * 64;  // fragments of one K-wave and row block
    if (nthr > per_q && p.split_k > 1 && !p.two_pass) {
        const float *sf = reinterpret_cast<const float *>(stash);
        const int lo = lane & 15, hi = lane >> 4;
        for (int b = 0; b < w.nblk; ++b) {
            const int rb = w.rb0 + b * w.rbs;
            int bst = bst0, bcnt = bcnt0;
            if (b > 0) block_rows(p, rb, bst, bcnt);
#pragma unroll
            for (int t = 0; t < G; ++t) {
                const int rl = 16 * G * wn + 16 * t + lo;
                const int fb = ((b * p.waves_k * p.waves_n + wn) * G + t) * MT;
                for (int m = hi + 4 * wk; m < p.M; m += 4 * p.waves_k) {
                    // fragment (b, q, wn, t, m / 16), lane 16 ((m & 15) / 4) + lo, element m & 3
                    const int f0 = fb + (m >> 4);
                    const int el = (16 * ((m & 15) >> 2) + lo) * 4 + hi;
                    float v = sf[f0 * 256 + el];
                    for (int q = 1; q < p.waves_k; ++q)
                        v += sf[(f0 + q * p.waves_n * G * MT) * 256 + el];
                    finish_output(p, w, rb, bst, bcnt, m, rl, v);
                }
            }
        }
        return;
    }
    for (int b = 0; b < w.nblk; ++b) {
        const int rb = w.rb0 + b * w.rbs;
        int bst = bst0, bcnt = bcnt0;
        if (b > 0) block_rows(p, rb, bst, bcnt);
        for (int e = threadIdx.x; e < per_q; e += nthr) {
            const f32x4_t *src = stash + (size_t)b * p.waves_k * per_q + e;
            f32x4_t v = src[0];
            for (int q = 1; q < p.waves_k; ++q) v += src[q * per_q];
            const int lane = e & 63;
            const int r = e >> 6;
            const int mt = r % MT;
            const int tt = (r / MT) % G;
            const int wn = r / (MT * G);
            const int rlf = 16 * G * wn + 16 * tt + (lane & 15);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int m = 16 * mt + 4 * (lane >> 4) + j;
                if (m < p.M) finish_output(p, w, rb, bst, bcnt, m, rlf, v[j]);
            }
        }
    }
}

// One row block per workgroup, no K split across workgroups, and at most two
// fragments per wave position (G MT <= 2): each wave of K-wave 0 takes the
// fragments of its own N-wave position at its own lanes, with the fragment
// indices known at compile time and the stores inline (the same sums, in the
// same order).  Measured on the deep projection at M = 16: 0.3 us less after
// the stream than the general mapping.
template <int G, int MT>
__device__ __forceinline__ void write_block_kwave0(const KParams &p, const f32x4_t *stash,
                                                   int wk, int wn, int lane, int bst, int bcnt) {
    __syncthreads();
    if (wk != 0) return;
    const int per_q = p.waves_n * G * MT * 64;  // f32x4 per K-wave
    const f32x4_t *src = stash + wn * G * MT * 64 + lane;
    const int rlw = wn * (16 * G) + (lane & 15);
#pragma unroll
    for (int t = 0; t < G; ++t) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            f32x4_t v = src[(t * MT + mt) * 64];
            for (int q = 1; q < p.waves_k; ++q) v += src[q * per_q + (t * MT + mt) * 64];
            const int rl = rlw + 16 * t;
            if (rl < bcnt) store_c4(p, 16 * mt + 4 * (lane >> 4), bst + rl, v);
        }
    }
}

// Barrier after staging A with direct-to-LDS loads that were issued before
// the NV newest vector memory operations of this wave: waits for everything
// older than those (vmcnt) and for this wave's LDS stores (lgkmcnt), then
// meets the other waves.  A fence over LDS here would make the compiler wait
// for every outstanding load (it cannot tell the staging loads from the
// ring's), so only compiler-level fences keep LDS accesses on their side.
template <int NV>
__device__ __forceinline__ void staged_barrier();

// s_waitcnt that waits until at most n vector memory operations of this wave
// are outstanding (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt and
// lgkmcnt left at their no-wait maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// The same with a run-time count: waits until at most r * L are outstanding
// (0 <= r < R; r is wave-uniform).
template <int L, int R>
__device__ __forceinline__ void wait_vmcnt_steps(int r) {
    if constexpr (R > 0) {
        if (r == R - 1)
            wait_vmcnt<(R - 1) * L>();
        else
            wait_vmcnt_steps<L, R - 1>(r);
    }
}

// Waits until at most min(PF - 1, r) * LB + min(PF - 2, r) * LA vector memory
// operations are outstanding, r = min(left, R - 1) (left wave-uniform).
template <int LB, int LA, int PF, int R>
__device__ __forceinline__ void wait_ring_left(int left) {
    if constexpr (R <= 1) {
        wait_vmcnt<0>();
    } else {
        constexpr int r = R - 1;
        if (left >= r)
            wait_vmcnt<(r < PF - 1 ? r : PF - 1) * LB + (r < PF - 2 ? r : PF - 2) * LA>();
        else
            wait_ring_left<LB, LA, PF, R - 1>(left);
    }
}

template <int NV>
__device__ __forceinline__ void staged_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    wait_vmcnt<NV>();
    __builtin_amdgcn_s_waitcnt((0x3F & 0xF) | ((0x3F >> 4) << 14) | (0x7 << 4) | (0x0 << 8));
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ---- VALU kernel --------------------------------------------------------------
// M: tokens (compile time); R: row slots per wave (4 rows each);
// PF: K-steps of B loads in flight (register ring depth); AG: each step's
// activation chunks are loaded from global memory (L2-resident) into the same
// ring as B, instead of being staged in LDS before the stream (no staging
// latency and no barrier; M more loads per step).  WF: the weights are fp32
// (p.B points to fp32 rows of p.ldb elements): a lane's chunk of eight k is
// then 32 bytes of a row, read as two 16-byte loads from the same window,
// and each product is one fp32 fused multiply-add of the widened activation.
template <int M, int R, int PF, bool AG, bool WF = false>
__global__ void __launch_bounds__(kMaxWaves * 64) skg_valu_kernel(KParams p) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    uint16_t *As = reinterpret_cast<uint16_t *>(smem);
    float *stash = reinterpret_cast<float *>(smem + p.stash_offset);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int l16 = lane & 15;
    const int slot = lane >> 4;
    const int wk = wave / p.waves_n;
    const int wn = wave - wk * p.waves_n;
    const WgPlan w = wg_plan(p);
    const int NB = p.rows_per_wg;
    const int SPB = p.wave_chunks / kValuStep;  // K steps per row block
    const int T = w.nblk * SPB;
    const int wv_c0 = w.wg_c0 + wk * p.wave_chunks;
    // first step of the slice that reaches past the last full chunk
    const int tail_st = max(0, (p.nfull - wv_c0) / kValuStep);
    const int rl0 = wn * (4 * R) + slot;  // local row of slot r = 0

    // load cursor: row block lb, step lst; once past the last row block the
    // loads read row 0 of A instead (in bounds, cache-resident, never used;
    // with fp32 weights row 0 of B, which holds the 2K bytes such a load
    // may reach)
    constexpr int WL = WF ? 2 : 1;  // 16-byte loads per row and step
    int lb = 0, lst = 0;
    const uint16_t *rowp[R];  // row starts, in 16-bit units
    auto set_rows = [&](int b) {
        int bst = 0, bcnt = 1;
        if (b < w.nblk) block_rows(p, w.rb0 + b * w.rbs, bst, bcnt);
#pragma unroll
        for (int r = 0; r < R; ++r)
            rowp[r] = (b < w.nblk)
                          ? p.B + (int64_t)(bst + min(rl0 + 4 * r, bcnt - 1)) * p.ldb * WL
                          : (WF ? p.B : p.A);
    };
    constexpr int NA = AG ? M : 1;
    auto issue = [&](uint4(&dst)[R][WL], uint4(&adst)[NA]) {
        const int64_t off = window_off(wv_c0 + lst * kValuStep + l16, p);
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int h = 0; h < WL; ++h) dst[r][h] = ldg16_stream(rowp[r] + WL * off + 8 * h);
        if constexpr (AG)
#pragma unroll
            for (int m = 0; m < M; ++m) adst[m] = ldg16(p.A + (int64_t)m * p.lda + off);
        if (++lst == SPB) {
            lst = 0;
            set_rows(++lb);
        }
    };

    uint4 buf[PF][R][WL];
    uint4 abuf[PF][NA];
    set_rows(0);
    if constexpr (AG) {
#pragma unroll
        for (int i = 0; i < PF; ++i) issue(buf[i], abuf[i]);
    } else {
        // A is staged first, so waiting for it (the oldest loads) leaves the
        // ring's loads in flight
        stage_a(p, As, w.wg_c0);
#pragma unroll
        for (int i = 0; i < PF; ++i) issue(buf[i], abuf[i]);
        staged_barrier<PF * R * WL>();
    }

    // rows of the first row block, for its end, computed while the first
    // loads are on their way: the empty statement keeps the compiler from
    // moving the division to the end of the stream, and holds the two
    // (workgroup-uniform) values in scalar registers meanwhile
    int bst0 = 0, bcnt0 = 0;
    if (w.nblk > 0) block_rows(p, w.rb0, bst0, bcnt0);
    __asm__ volatile("" : "+s"(bst0), "+s"(bcnt0));

    float acc[R][M];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;

    constexpr int VP = Pow2Ceil<M>::v;
    const bool writer = l16 < M;
    const uint16_t *ap = As + (wk * p.wave_chunks + l16) * kChunk;
    // stash: [row block][K-wave][m][local row]
    const int per_block = p.waves_k * M * NB;
    const bool direct = direct_write(p);

    int cb = 0, cst = 0;  // compute cursor
    auto step = [&](uint4(&bv)[R][WL], uint4(&av)[NA]) {
        if (cst >= tail_st) {
            const int c = wv_c0 + cst * kValuStep + l16;
            const uint4 mk = tail_mask(c, p);
            if constexpr (WF) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint4 mw = tail_mask_f32(c, p, h);
#pragma unroll
                    for (int r = 0; r < R; ++r) bv[r][h] = and4(bv[r][h], mw);
                }
            } else {
#pragma unroll
                for (int r = 0; r < R; ++r) bv[r][0] = and4(bv[r][0], mk);
            }
            if constexpr (AG)
#pragma unroll
                for (int m = 0; m < M; ++m) av[m] = and4(av[m], mk);
        }
        uint4 a[M];
        if constexpr (AG) {
#pragma unroll
            for (int m = 0; m < M; ++m) a[m] = av[m];
        } else {
            const uint16_t *a_st = ap + cst * (kValuStep * kChunk);
#pragma unroll
            for (int m = 0; m < M; ++m) a[m] = lds16(a_st + m * p.lds_stride);
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < M; ++m) {
                if constexpr (WF)
                    acc[r][m] = dot8_f32w(a[m], bv[r][0], bv[r][1], acc[r][m]);
                else
                    acc[r][m] = dot8(a[m], bv[r][0], acc[r][m]);
            }
        if (++cst == SPB) {
            // row block done: lane m of each row group now takes token m
            const int rb = w.rb0 + cb * w.rbs;
            int bst = bst0, bcnt = bcnt0;
            if (cb > 0) block_rows(p, rb, bst, bcnt);
            float *dst = stash + cb * per_block + (wk * M + l16) * NB + rl0;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                float v[VP];
#pragma unroll
                for (int j = 0; j < VP; ++j) v[j] = (j < M) ? acc[r][j] : 0.0f;
                reduce16<VP>(v, lane);
                if (writer) {
                    if (!direct) {
                        dst[4 * r] = v[0];
                    } else if (p.split_k == 1) {
                        if (rl0 + 4 * r < bcnt) store_c(p, l16, bst + rl0 + 4 * r, v[0]);
                    } else {
                        p.ws[((size_t)(rb * p.split_k + w.s) * M + l16) * NB + rl0 + 4 * r] = v[0];
                    }
                }
#pragma unroll
                for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;
            }
            cst = 0;
            ++cb;
        }
    };

    // Whole rounds of the ring: every slot is refilled unconditionally right
    // after it is consumed, so the compiler keeps each slot in the same
    // registers and waits for exactly that slot's loads.  The last round only
    // consumes; refills for steps past T read A (see set_rows).  Refilling
    // only while steps remain (no load left in flight at the end, as the LDS
    // ring does) measured slower in this register ring, e.g. 8.34 -> 10.63 us
    // on a 2 x 7168 x 2112 product; our reading is that the compiler's waits
    // where the conditional refills join cover more loads than the slot's.
    const int TT = (T + PF - 1) / PF * PF;
    int t0 = 0;
    for (; t0 + PF < TT; t0 += PF) {
#pragma unroll
        for (int i = 0; i < PF; ++i) {
            if (t0 + i < T) step(buf[i], abuf[i]);
            issue(buf[i], abuf[i]);
        }
    }
#pragma unroll
    for (int i = 0; i < PF; ++i)
        if (t0 + i < T) step(buf[i], abuf[i]);
    if (!direct) write_blocks<R>(p, w, stash, bst0, bcnt0, wk, wn, lane);
}

// ---- MFMA kernel ------------------------------------------------------------
// Stage A[:, slice] in LDS in MFMA operand order: for each 32-wide K step, the
// 64 lane fragments (lane l: token m = l & 15, chunk l >> 4 of the step) lie
// contiguously, so the per-step operand read is one conflict-free 1 KB
// ds_read_b128.  One direct-to-LDS load per step block; tokens m >= M load
// row M-1 (the readers mask them to zero); chunks at or beyond K are written
// as (partial) zeros by ordinary LDS stores.
// (RAW: through lds_dma16_raw, for kernels whose other LDS writes by DMA the
// compiler does not see either; their barrier waits for these loads)
// MT token tiles of 16 (M up to 16 MT): the 1 KB blocks of one 32-wide step
// follow each other, tile mt holding tokens 16 mt .. 16 mt + 15.
template <bool RAW = false, int MT = 1>
__device__ __forceinline__ void stage_a_frag(const KParams &p, uint16_t *As, int wg_c0) {
    const int lane = threadIdx.x & 63;
    const int nwaves = p.waves_n * p.waves_k;
    const int nblk = (p.wg_chunks >> 2) * MT;  // (32-wide step, token tile) blocks
    for (int blk = threadIdx.x >> 6; blk < nblk; blk += nwaves) {
        const int mt = blk % MT;
        const int m = min(16 * mt + (lane & 15), p.M - 1);
        const uint16_t *rowp = p.A + (int64_t)m * p.lda;
        const int c = wg_c0 + 4 * (blk / MT) + (lane >> 4);
        uint16_t *dst = As + blk * 64 * kChunk;
        if (c < p.nfull) {
            if constexpr (RAW)
                lds_dma16_raw<false>(rowp + (int64_t)c * kChunk, lds_addr_of(dst));
            else
                lds_dma16(rowp + (int64_t)c * kChunk, dst);
        } else {
            sts16(dst + lane * kChunk, load_chunk_tail(rowp, c, p));
        }
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

// G: 16-row tiles per wave; PF: 128-wide K steps of loads in flight; AQ: 0
// when the activations are staged in LDS, else the number of activation loads
// per step and token tile (rows 4q + (lane >> 4), q < AQ: AQ = 4 covers 16
// tokens, AQ = 2 covers M <= 8): the activations are then loaded from global
// memory (L2-resident), in the same ring and row-segment layout as B, and
// transposed through their own wave-private tiles.  MT: token tiles of 16
// (M <= 16 MT at run time; MT > 1 takes AQ = 4), each its own 16-row MFMA
// operand against the same B tiles.  Activation rows m >= M are fed as zeros.
template <int G, int PF, int AQ, int MT = 1>
__global__ void __launch_bounds__(kMaxWaves * 64) skg_mfma_kernel(KParams p) {
    constexpr bool AG = AQ > 0;
    static_assert(MT == 1 || AQ == 0 || AQ == 4, "several token tiles load whole tiles");
    constexpr int NA = AG ? MT * AQ : 1;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    uint16_t *As = reinterpret_cast<uint16_t *>(smem);
    float *stash = reinterpret_cast<float *>(smem + p.stash_offset);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
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
    const int tail_st = max(0, (p.nfull - wv_c0) / kValuStep);
    constexpr int NT = G + (AG ? MT : 0);  // transpose tiles per wave (B tiles, then A)
    uint4 *tile = reinterpret_cast<uint4 *>(smem + p.tr_offset) + wave * (NT * 256);
    // AG: activation rows 4q + hi of this lane, A tile q / 4 (rows >= M read
    // row M-1, masked)
    const uint16_t *arow[NA];
    uint4 amask[NA];
#pragma unroll
    for (int q = 0; q < NA; ++q) {
        arow[q] = p.A + (int64_t)min(4 * q + hi, M - 1) * p.lda;
        const uint32_t mq = (4 * q + hi < M) ? 0xFFFFFFFFu : 0u;
        amask[q] = make_uint4(mq, mq, mq, mq);
    }

    // load cursor; past the last row block the B loads read row 0 of A
    int lb = 0, lst = 0;
    const uint16_t *rowp[G][4];
    auto set_rows = [&](int b) {
        int bst = 0, bcnt = 1;
        if (b < w.nblk) block_rows(p, w.rb0 + b * w.rbs, bst, bcnt);
        const int rl = wn * (16 * G) + hi;
#pragma unroll
        for (int t = 0; t < G; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                rowp[t][q] = (b < w.nblk)
                                 ? p.B + (int64_t)(bst + min(rl + 16 * t + 4 * q, bcnt - 1)) * p.ldb
                                 : p.A;
    };
    auto issue = [&](uint4(&dst)[G][4], uint4(&adst)[NA]) {
        const int64_t off = window_off(wv_c0 + lst * kValuStep + lo, p);
#pragma unroll
        for (int t = 0; t < G; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q) dst[t][q] = ldg16_stream(rowp[t][q] + off);
        if constexpr (AG)
#pragma unroll
            for (int q = 0; q < NA; ++q) adst[q] = ldg16(arow[q] + off);
        if (++lst == SPB) {
            lst = 0;
            set_rows(++lb);
        }
    };

    uint4 buf[PF][G][4];
    uint4 abuf[PF][NA];
    set_rows(0);
    if constexpr (!AG) stage_a_frag<false, MT>(p, As, w.wg_c0);  // oldest loads, as in the VALU kernel
#pragma unroll
    for (int i = 0; i < PF; ++i) issue(buf[i], abuf[i]);

    if constexpr (!AG) {
        staged_barrier<PF * G * 4>();
    } else {
        // activation rows 4 * AQ .. 15 of the A tile stay zero
#pragma unroll
        for (int q = AQ; q < 4; ++q)
            tile[G * 256 + tile_slot(4 * q + hi, lo)] = make_uint4(0u, 0u, 0u, 0u);
    }

    f32x4_t acc[G][MT];
#pragma unroll
    for (int t = 0; t < G; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // LDS activation fragments of this wave: MT 1 KB blocks per 32-wide step;
    // lanes of tokens m >= M zero what they read
    const uint16_t *ap = As + ((wk * p.wave_chunks) / 4 * MT * 64 + lane) * kChunk;
    uint32_t lane_mask[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) lane_mask[mt] = (16 * mt + lo < M) ? 0xFFFFFFFFu : 0u;
    // stash: [row block][K-wave][N-wave][tile][token tile] blocks of 64 lanes x
    // 4 floats; lane 16*hi + lo, element v holds token 16*mt + 4*hi + v, row
    // 16*tile + lo
    f32x4_t *st = reinterpret_cast<f32x4_t *>(stash) + (wk * p.waves_n + wn) * G * MT * 64 + lane;
    const int st_block = p.waves_k * p.waves_n * G * MT * 64;  // f32x4 per row block
    const bool direct = direct_write(p);
    const int rlw = wn * (16 * G);  // first local row of this wave

    int cb = 0, cst = 0;
    auto step = [&](uint4(&bv)[G][4], uint4(&av)[NA]) {
        if (cst >= tail_st) {
            const uint4 mk = tail_mask(wv_c0 + cst * kValuStep + lo, p);
#pragma unroll
            for (int t = 0; t < G; ++t)
#pragma unroll
                for (int q = 0; q < 4; ++q) bv[t][q] = and4(bv[t][q], mk);
            if constexpr (AG)
#pragma unroll
                for (int q = 0; q < AQ; ++q) av[q] = and4(av[q], mk);
        }
        // transpose this step's B (and A) through the wave's LDS tiles
#pragma unroll
        for (int t = 0; t < G; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q) tile[t * 256 + tile_slot(4 * q + hi, lo)] = bv[t][q];
        if constexpr (AG)
#pragma unroll
            for (int q = 0; q < NA; ++q)
                tile[(G + q / 4) * 256 + tile_slot(4 * (q % 4) + hi, lo)] = and4(av[q], amask[q]);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            bf16x8_t a8[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                uint4 a;
                if constexpr (AG) {
                    a = tile[(G + mt) * 256 + tile_slot(lo, 4 * s + hi)];
                } else {
                    a = lds16(ap + ((cst * 4 + s) * MT + mt) * (64 * kChunk));
                    a.x &= lane_mask[mt];
                    a.y &= lane_mask[mt];
                    a.z &= lane_mask[mt];
                    a.w &= lane_mask[mt];
                }
                a8[mt] = __builtin_bit_cast(bf16x8_t, a);
            }
#pragma unroll
            for (int t = 0; t < G; ++t) {
                const uint4 b8 = tile[t * 256 + tile_slot(lo, 4 * s + hi)];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    acc[t][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        a8[mt], __builtin_bit_cast(bf16x8_t, b8), acc[t][mt], 0, 0, 0);
            }
        }
        if (++cst == SPB) {
            // acc[t][v] holds token 4*hi + v of local row rlw + 16*t + lo
            const int rb = w.rb0 + cb * w.rbs;
            int bst, bcnt;
            block_rows(p, rb, bst, bcnt);
#pragma unroll
            for (int t = 0; t < G; ++t) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    if (!direct) {
                        st[cb * st_block + (t * MT + mt) * 64] = acc[t][mt];
                    } else {
                        // lane index re-derived here so the compiler cannot
                        // keep the store addresses live across the whole stream
                        int ln = lane;
                        __asm__ volatile("" : "+v"(ln));
                        const int rl = rlw + 16 * t + (ln & 15);
                        if (p.split_k == 1) {
                            if (rl < bcnt) store_c4(p, 16 * mt + 4 * (ln >> 4), bst + rl, acc[t][mt]);
                        } else {
#pragma unroll
                            for (int v = 0; v < 4; ++v) {
                                const int m = 16 * mt + 4 * (ln >> 4) + v;
                                if (m < M)
                                    p.ws[((size_t)(rb * p.split_k + w.s) * M + m) * NB + rl] =
                                        acc[t][mt][v];
                            }
                        }
                    }
                    acc[t][mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
                }
            }
            cst = 0;
            ++cb;
        }
    };

    // Whole rounds of the ring, as in the VALU kernel, but the last round
    // refills too (from A): a separate last round costs this kernel more
    // registers than the few extra cache-resident loads cost time.
    const int TT = (T + PF - 1) / PF * PF;
    for (int t0 = 0; t0 < TT; t0 += PF) {
#pragma unroll
        for (int i = 0; i < PF; ++i) {
            if (t0 + i < T) step(buf[i], abuf[i]);
            issue(buf[i], abuf[i]);
        }
    }
    if (!direct) {
        int bst0 = 0, bcnt0 = 0;
        if (w.nblk > 0) block_rows(p, w.rb0, bst0, bcnt0);
        write_blocks_frag<G, MT>(p, w, reinterpret_cast<const f32x4_t *>(stash), bst0, bcnt0, wk,
                                 wn, lane);
    }
}

// ---- MFMA kernel with an LDS ring --------------------------------------------
// Same tiles, operands and epilogue as skg_mfma_kernel, but the loads write
// straight into the wave's LDS tiles (global_load_lds_dwordx4) instead of a
// register ring: a DMA instruction puts lane l's 16 bytes in slot l of a 1 KB
// block (rows 4q .. 4q + 3 of the tile), so lane l fetches the chunk that
// belongs in that slot of the XOR-swizzled tile, chunk (l & 15) ^ r of row
// r = 4q + (l >> 4).  Each quarter-wave still reads one 256-byte row segment
// (in permuted lane order), the tile needs no transposing writes, and the
// ring costs LDS rather than VGPRs.  PF ring slots of G B tiles (plus one
// activation tile when AQ > 0) per wave; K-tail masks are applied to the
// operands as they are read.  Tokens m >= M read row M - 1 of A and produce
// accumulator rows that are never stored (an MFMA output row depends on its
// own activation row only).
// SY (with activations loaded per step, AQ > 0): 0, the waves run freely; 1,
// the workgroup's waves meet at a barrier every K step (their loads of
// neighbouring rows at the same K then reach memory together, measured
// faster on some shapes); 2, as 1, and each step's activation tile is loaded
// once per workgroup (by the waves with wn == 0, one per K-wave group) into a
// ring the waves share, instead of once per wave.  A shared slot can only be
// refilled when every wave has read it, i.e. after the next step's barrier,
// so the shared ring runs one step behind the weights' (depth >= 3 keeps
// depth - 2 activation steps in flight); each wave's weights are refilled
// right after it reads them, as in the other kinds.  Every wave of a
// workgroup runs the same number of steps, so all of them reach every
// barrier.
template <int G, int PF, int AQ, int MT = 1, int SY = 0>
__global__ void __launch_bounds__(kMaxWaves * 64) skg_mfma_ring_kernel(KParams p) {
    constexpr bool AG = AQ > 0;
    constexpr bool SH = SY == 2;
    static_assert(MT == 1 || AQ == 0 || AQ == 4, "several token tiles load whole tiles");
    static_assert(SY == 0 || (AG && MT == 1), "barrier modes take per-step activations, M <= 16");
    static_assert(!SH || PF >= 3, "a shared ring needs depth >= 3");
    constexpr int NT = G + ((AG && !SH) ? MT : 0);  // tiles per ring slot of a wave
    constexpr int LB = 4 * G;                        // weight loads per K step
    constexpr int L = LB + MT * AQ;                  // loads per K step with the activations
    static_assert((PF - 1) * L < 64 && PF * L < 64, "vmcnt range");
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    uint16_t *As = reinterpret_cast<uint16_t *>(smem);
    float *stash = reinterpret_cast<float *>(smem + p.stash_offset);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lo = lane & 15;
    const int hi = lane >> 4;
    const int wk = wave / p.waves_n;
    const int wn = wave - wk * p.waves_n;
    const WgPlan w = wg_plan(p);
    const int NB = p.rows_per_wg;
    const int M = p.M;
    const int SPB = p.wave_chunks / kValuStep;
    const int T = w.nblk * SPB;
    const int wv_c0 = w.wg_c0 + wk * p.wave_chunks;
    const int tail_st = max(0, (p.nfull - wv_c0) / kValuStep);
    uint4 *ring = reinterpret_cast<uint4 *>(smem + p.tr_offset) + wave * (PF * NT * 256);
    // SY = 2: the shared activation ring after all waves' rings, slot s of
    // K-wave group wk at tile (s * waves_k + wk); loaded by the wn == 0 waves
    const uint4 *aring = reinterpret_cast<const uint4 *>(smem + p.tr_offset) +
                         p.waves_n * p.waves_k * (PF * NT * 256);
    const bool loader = !SH || wn == 0;
    // chunk of the step fetched by this lane for DMA block q
    int swz[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) swz[q] = lo ^ (4 * q + hi);
    const uint16_t *arow[AG ? MT * AQ : 1];
#pragma unroll
    for (int q = 0; q < (AG ? MT * AQ : 1); ++q)
        arow[q] = p.A + (int64_t)min(4 * q + hi, M - 1) * p.lda;

    int lb = 0, lst = 0;
    const uint16_t *rowp[G][4];
    auto set_rows = [&](int b) __attribute__((always_inline)) {
        int bst = 0, bcnt = 1;
        if (b < w.nblk) block_rows(p, w.rb0 + b * w.rbs, bst, bcnt);
        const int rl = wn * (16 * G) + hi;
#pragma unroll
        for (int t = 0; t < G; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                rowp[t][q] = (b < w.nblk)
                                 ? p.B + (int64_t)(bst + min(rl + 16 * t + 4 * q, bcnt - 1)) * p.ldb
                                 : p.A;
    };
    const uint32_t ring_addr = lds_addr_of(ring);
    const uint32_t aring_addr = lds_addr_of(aring);
    auto issue = [&](int slot) __attribute__((always_inline)) {
        const uint32_t dst = ring_addr + slot * (NT * kTileBytes);
        const uint32_t adst = dst + G * kTileBytes;  // the wave's own activation tiles
        const int cb0 = wv_c0 + lst * kValuStep;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t off = window_off(cb0 + swz[q], p);
#pragma unroll
            for (int t = 0; t < G; ++t)
                lds_dma16_raw<true>(rowp[t][q] + off, dst + t * kTileBytes + 1024 * q);
            if constexpr (AG && !SH)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    if (q < AQ)
                        lds_dma16_raw<false>(arow[mt * AQ + q] + off,
                                             adst + mt * kTileBytes + 1024 * q);
        }
        if (++lst == SPB) {
            lst = 0;
            set_rows(++lb);
        }
    };
    // SY = 2, the loading waves: the activation tile of step u (its K range
    // depends on u's place in the row block only) into shared slot u % PF
    auto issue_a = [&](int u) __attribute__((always_inline)) {
        const uint32_t adst = aring_addr + ((u % PF) * p.waves_k + wk) * kTileBytes;
        const int cb0 = wv_c0 + (u % SPB) * kValuStep;
#pragma unroll
        for (int q = 0; q < AQ; ++q)
            lds_dma16_raw<false>(arow[q] + window_off(cb0 + swz[q], p), adst + 1024 * q);
    };

    set_rows(0);
    if constexpr (!AG) stage_a_frag<true, MT>(p, As, w.wg_c0);  // oldest loads
#pragma unroll
    for (int i = 0; i < PF; ++i) {
        issue(i);
        // the shared ring runs one step shorter (its slot is refilled after
        // the barrier that shows every wave has read it)
        if (SH && loader && i < PF - 1) issue_a(i);
    }
    if constexpr (!AG) staged_barrier<PF * L>();

    f32x4_t acc[G][MT];
#pragma unroll
    for (int t = 0; t < G; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    const uint16_t *ap = As + ((wk * p.wave_chunks) / 4 * MT * 64 + lane) * kChunk;
    f32x4_t *st = reinterpret_cast<f32x4_t *>(stash) + (wk * p.waves_n + wn) * G * MT * 64 + lane;
    const int st_block = p.waves_k * p.waves_n * G * MT * 64;
    const bool direct = direct_write(p);
    const int rlw = wn * (16 * G);
    // rows of the first row block, for its end, computed while the first
    // loads are on their way: the empty statement keeps the compiler from
    // moving the division to the end of the stream, and holds the two
    // (workgroup-uniform) values in scalar registers meanwhile
    int bst0 = 0, bcnt0 = 0;
    if (w.nblk > 0) block_rows(p, w.rb0, bst0, bcnt0);
    __asm__ volatile("" : "+s"(bst0), "+s"(bcnt0));

    int cb = 0, cst = 0;
    // the workgroup's waves meet (their earlier LDS reads complete first)
    auto meet = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt((0x3F & 0xF) | ((0x3F >> 4) << 14) | (0x7 << 4) | (0x0 << 8));
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
    };
    auto compute = [&](int slot) __attribute__((always_inline)) {
        const uint4 *tl = ring + slot * (NT * 256);
        const uint4 *atl = SH ? aring + (slot * p.waves_k + wk) * (MT * 256) : tl + G * 256;
        // all operands first, so the reads go out back to back
        uint4 av[4][MT], bv[4][G];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                av[s][mt] = AG ? atl[mt * 256 + tile_slot(lo, 4 * s + hi)]
                               : lds16(ap + ((cst * 4 + s) * MT + mt) * (64 * kChunk));
#pragma unroll
            for (int t = 0; t < G; ++t) bv[s][t] = tl[t * 256 + tile_slot(lo, 4 * s + hi)];
        }
        if (cst >= tail_st) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const uint4 mk = tail_mask(wv_c0 + cst * kValuStep + 4 * s + hi, p);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) av[s][mt] = and4(av[s][mt], mk);
#pragma unroll
                for (int t = 0; t < G; ++t) bv[s][t] = and4(bv[s][t], mk);
            }
        }
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int t = 0; t < G; ++t)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    acc[t][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, av[s][mt]),
                        __builtin_bit_cast(bf16x8_t, bv[s][t]), acc[t][mt], 0, 0, 0);
        if (++cst == SPB) {
            const int rb = w.rb0 + cb * w.rbs;
            int bst = bst0, bcnt = bcnt0;
            if (cb > 0) block_rows(p, rb, bst, bcnt);
#pragma unroll
            for (int t = 0; t < G; ++t) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    if (!direct) {
                        st[cb * st_block + (t * MT + mt) * 64] = acc[t][mt];
                    } else {
                        // lane index re-derived here so the compiler cannot
                        // keep the store addresses live across the whole stream
                        int ln = lane;
                        __asm__ volatile("" : "+v"(ln));
                        const int rl = rlw + 16 * t + (ln & 15);
                        if (p.split_k == 1) {
                            if (rl < bcnt) store_c4(p, 16 * mt + 4 * (ln >> 4), bst + rl, acc[t][mt]);
                        } else {
#pragma unroll
                            for (int v = 0; v < 4; ++v) {
                                const int m = 16 * mt + 4 * (ln >> 4) + v;
                                if (m < M)
                                    p.ws[((size_t)(rb * p.split_k + w.s) * M + m) * NB + rl] =
                                        acc[t][mt][v];
                            }
                        }
                    }
                    acc[t][mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
                }
            }
            cst = 0;
            ++cb;
        }
    };
    auto step = [&](int slot, int left) __attribute__((always_inline)) {
        // this slot's loads are the oldest; the later steps (PF - 1 of them,
        // or the `left` steps still to come near the end) stay in flight
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (left >= PF - 1)
            wait_vmcnt<(PF - 1) * L>();
        else
            wait_vmcnt_steps<L, PF - 1>(left);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if constexpr (SY == 1) meet();
        compute(slot);
    };

    if constexpr (SH) {
        // Issue order B(0) A(0) B(1) A(1) ...: a wave's weights B(u) for step
        // u are refilled right after it reads slot u - PF, as in the other
        // kinds; the activations A(u) only after the barrier of step u - PF +
        // 1.  Behind A(t) (a loading wave) there are then min(PF - 1, left)
        // weight steps and min(PF - 2, left) activation steps, left = T - 1 -
        // t; behind B(t) (the other waves) min(PF - 1, left) weight steps.
        for (int t = 0; t < T; ++t) {
            const int left = T - 1 - t;
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            if (loader)
                wait_ring_left<LB, MT * AQ, PF, PF>(left);
            else
                wait_ring_left<LB, 0, PF, PF>(left);
            meet();
            if (loader && t + PF - 1 < T) issue_a(t + PF - 1);
            compute(t % PF);
            if (t + PF < T) issue(t % PF);
        }
    } else {
    // whole rounds: every slot is refilled right after it is read, as long as
    // steps remain (no load is issued that the wave does not consume, so the
    // last step's wait is the wave's last).  The rounds in which every step
    // refills run without the end-of-stream checks.
    const int TT = (T + PF - 1) / PF * PF;
    int t0 = 0;
    for (; t0 + 2 * PF <= T; t0 += PF) {
#pragma unroll
        for (int i = 0; i < PF; ++i) {
            step(i, PF - 1);
            issue(i);
        }
    }
    for (; t0 < TT; t0 += PF) {
#pragma unroll
        for (int i = 0; i < PF; ++i) {
            if (t0 + i < T) step(i, T - 1 - (t0 + i));
            if (t0 + i + PF < T) issue(i);
        }
    }
    }
    // no LDS write may still be on its way when the workgroup's LDS is reused
    wait_vmcnt<0>();
    if constexpr (G * MT <= 2) {
        if (!direct && p.split_k == 1 && w.nblk == 1) {
            write_block_kwave0<G, MT>(p, reinterpret_cast<const f32x4_t *>(stash), wk, wn, lane,
                                      bst0, bcnt0);
            return;
        }
    }
    if (!direct)
        write_blocks_frag<G, MT>(p, w, reinterpret_cast<const f32x4_t *>(stash), bst0, bcnt0, wk,
                                 wn, lane);
}

// Over fp32 weights the register ring is twice as large, and these
// (M, rows, depth) combinations would spill to scratch (measured with the
// compiler's resource-usage report), so they are not built: the largest M
// per (R, PF), with activations staged in LDS (AG false) or in the ring.
constexpr int f32w_max_m(int R, int PF, bool AG) {
    return !AG ? ((R == 4 && PF == 4) ? 8 : (R == 2 && PF == 8) ? 10 : (R == 4 && PF == 2) ? 12 : 16)
               : ((PF == 12 || (R == 2 && PF == 8)) ? 2 : (R == 4 && PF == 4) ? 4
                  : (R == 1 && PF == 8) ? 5 : (R == 2 && PF == 4) ? 7 : 8);
}

template <int M, int R, int PF, bool AG>
constexpr KernelPtr f32w_kernel() {
    if constexpr (M <= f32w_max_m(R, PF, AG))
        return skg_valu_kernel<M, R, PF, AG, true>;
    else
        return nullptr;
}

// Over bf16 weights with the activation chunks in the load ring (AG), the
// ring holds M extra loads per step. Configurations with M * depth > 32 are
// rejected by the configuration check, and 8 tokens with 4 rows at depth 4
// spill to scratch (the code object's metadata report a private segment), so
// none of these is built: the largest M per (R, PF).
constexpr int bf16_ga_max_m(int R, int PF) {
    return (R == 4 && PF == 4) ? 7 : (32 / PF < 8 ? 32 / PF : 8);
}

template <int M, int R, int PF>
constexpr KernelPtr bf16_ga_kernel() {
    if constexpr (M <= bf16_ga_max_m(R, PF))
        return skg_valu_kernel<M, R, PF, true>;
    else
        return nullptr;
}

// Instantiation list for one M, in the order of kValuVariants (bf16
// weights, activations staged in LDS; SKG_VALU_ROW_GA: activations in the
// ring; SKG_VALU_ROW_F32W: fp32 weights; nullptr where not built).
#define SKG_VALU_ROW(M, AG)                                                              \
    {skg_valu_kernel<M, 1, 4, AG>, skg_valu_kernel<M, 1, 8, AG>,                         \
     skg_valu_kernel<M, 1, 12, AG>, skg_valu_kernel<M, 2, 2, AG>,                        \
     skg_valu_kernel<M, 2, 4, AG>, skg_valu_kernel<M, 2, 8, AG>,                         \
     skg_valu_kernel<M, 4, 2, AG>, skg_valu_kernel<M, 4, 4, AG>}
#define SKG_VALU_ROW_GA(M)                                                               \
    {bf16_ga_kernel<M, 1, 4>(), bf16_ga_kernel<M, 1, 8>(),                               \
     bf16_ga_kernel<M, 1, 12>(), bf16_ga_kernel<M, 2, 2>(),                              \
     bf16_ga_kernel<M, 2, 4>(), bf16_ga_kernel<M, 2, 8>(),                               \
     bf16_ga_kernel<M, 4, 2>(), bf16_ga_kernel<M, 4, 4>()}
#define SKG_VALU_ROW_F32W(M, AG)                                                         \
    {f32w_kernel<M, 1, 4, AG>(), f32w_kernel<M, 1, 8, AG>(),                             \
     f32w_kernel<M, 1, 12, AG>(), f32w_kernel<M, 2, 2, AG>(),                            \
     f32w_kernel<M, 2, 4, AG>(), f32w_kernel<M, 2, 8, AG>(),                             \
     f32w_kernel<M, 4, 2, AG>(), f32w_kernel<M, 4, 4, AG>()}

}  // namespace
}  // namespace skg

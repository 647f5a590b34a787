// skg_launch.hip -- MFMA kernel instantiations, the zero-fill kernel, and
// the launch path shared by every variant.
#include <algorithm>
#include <mutex>
#include <set>
#include <utility>

#include "skg_device.h"

namespace skg {

namespace {

__global__ void skg_zero_fill_kernel(void *C, int M, int N, int64_t ldc, int out_bf16) {
    const int64_t total = (int64_t)M * N;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int m = (int)(i / N);
        const int n = (int)(i - (int64_t)m * N);
        if (out_bf16)
            reinterpret_cast<uint16_t *>(C)[(int64_t)m * ldc + n] = 0;
        else
            reinterpret_cast<float *>(C)[(int64_t)m * ldc + n] = 0.0f;
    }
}

// K < 8: every row is shorter than one 16-byte window, so each output is a
// plain fp32 sum over k of elementwise products (one thread per output; the
// weights are bf16 or, with p.w_f32, fp32).
__global__ void skg_small_k_kernel(KParams p) {
    const int64_t total = (int64_t)p.M * p.N;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int m = (int)(i / p.N);
        const int n = (int)(i - (int64_t)m * p.N);
        const uint16_t *a = p.A + (int64_t)m * p.lda;
        float v = 0.0f;
        if (p.w_f32) {
            const float *b = reinterpret_cast<const float *>(p.B) + (int64_t)n * p.ldb;
            for (int k = 0; k < p.K; ++k)
                v = fmaf(__builtin_bit_cast(float, (uint32_t)a[k] << 16), b[k], v);
        } else {
            const uint16_t *b = p.B + (int64_t)n * p.ldb;
            for (int k = 0; k < p.K; ++k)
                v = fmaf(__builtin_bit_cast(float, (uint32_t)a[k] << 16),
                         __builtin_bit_cast(float, (uint32_t)b[k] << 16), v);
        }
        store_c(p, m, n, v);
    }
}

// Streaming read with the GEMM's load form (non-temporal 128-bit loads); each
// workgroup covers 8 x 4 KB contiguous per round and XOR-folds its words.
__global__ void __launch_bounds__(256) skg_stream_read_kernel(const uint16_t *src, size_t n16,
                                                              unsigned *sink) {
    __shared__ unsigned red[256];
    unsigned acc = 0;
    const size_t stride = (size_t)gridDim.x * blockDim.x * 8;
    for (size_t base = (size_t)blockIdx.x * blockDim.x * 8 + threadIdx.x; base < n16;
         base += stride) {
        uint4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const size_t i = base + (size_t)u * blockDim.x;
            v[u] = (i < n16) ? ldg16_stream(src + i * kChunk) : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) red[threadIdx.x] ^= red[threadIdx.x + s];
        __syncthreads();
    }
    if (threadIdx.x == 0) sink[blockIdx.x] = red[0];
}

// Second pass of SKG_BACKEND_SPLITK_2PASS: C[m][row] = sum over s (in split
// order) of ws[((rb*S + s)*M + m)*NB + rl], row = first row of block rb + rl
// (only rl < the block's row count); consecutive threads take
// consecutive rows, so partial reads and C writes are coalesced.
__global__ void skg_splitk_reduce_kernel(KParams p) {
    const int NB = p.rows_per_wg;
    const int per_rb = p.M * NB;
    const int64_t total = (int64_t)p.num_rb * per_rb;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int rb = (int)(i / per_rb);
        const int rem = (int)(i - (int64_t)rb * per_rb);
        const int m = rem / NB;
        const int rl = rem - m * NB;
        int bst, bcnt;
        block_rows(p, rb, bst, bcnt);
        if (rl < bcnt) {
            const float *src = p.ws + (size_t)rb * p.split_k * per_rb + rem;
            float v = 0.0f;
            for (int s = 0; s < p.split_k; ++s) v += src[(size_t)s * per_rb];
            store_c(p, m, bst + rl, v);
        }
    }
}

// The register ring with activations from L2 at 2 row tiles and depth 4
// spills to scratch over one full token tile (the code object's metadata
// report a private segment), so that combination is not built.
template <int G, int PF>
constexpr KernelPtr mfma_ga4_kernel() {
    if constexpr (G == 2 && PF == 4)
        return nullptr;
    else
        return skg_mfma_kernel<G, PF, 4>;
}

struct MfmaVariant {
    int G, PF;
    KernelPtr lds_a;  // activations staged in LDS
    KernelPtr ga2;    // activations loaded from global memory, M <= 8
    KernelPtr ga4;    // activations loaded from global memory, M <= 16 (one token tile)
    KernelPtr ring_lds_a, ring_ga2, ring_ga4;  // the same with the LDS ring
};
#define SKG_MFMA(G, PF)                                                                 \
    {G,                                                                                  \
     PF,                                                                                 \
     skg_mfma_kernel<G, PF, 0>,                                                          \
     skg_mfma_kernel<G, PF, 2>,                                                          \
     mfma_ga4_kernel<G, PF>(),                                                           \
     skg_mfma_ring_kernel<G, PF, 0>,                                                     \
     skg_mfma_ring_kernel<G, PF, 2>,                                                     \
     skg_mfma_ring_kernel<G, PF, 4>}
const MfmaVariant kMfmaVariants[] = {SKG_MFMA(1, 2), SKG_MFMA(1, 3), SKG_MFMA(1, 4),
                                     SKG_MFMA(1, 6), SKG_MFMA(2, 1), SKG_MFMA(2, 2),
                                     SKG_MFMA(2, 3), SKG_MFMA(2, 4), SKG_MFMA(4, 1),
                                     SKG_MFMA(4, 2)};
#undef SKG_MFMA
constexpr int kNumMfma = sizeof(kMfmaVariants) / sizeof(kMfmaVariants[0]);

KernelPtr find_kernel(int inner, int M, int row_tiles, int depth, bool f32w) {
    if (inner == SKG_INNER_VALU || inner == SKG_INNER_VALU_GA) {
        for (int i = 0; i < kNumValu; ++i)
            if (kValuVariants[i][0] == row_tiles && kValuVariants[i][1] == depth) {
                if (f32w) {
                    if (inner == SKG_INNER_VALU_GA)
                        return M <= 8 ? valu_kernel_f32w_ga(M, i) : nullptr;
                    return M <= 8 ? valu_kernel_f32w_lo(M, i) : valu_kernel_f32w_hi(M, i);
                }
                if (inner == SKG_INNER_VALU_GA) return M <= 8 ? valu_kernel_ga(M, i) : nullptr;
                return M <= 8 ? valu_kernel_lo(M, i) : valu_kernel_hi(M, i);
            }
        return nullptr;
    }
    if (f32w) return nullptr;  // matrix-core kernels take bf16 weights only
    if (inner == SKG_INNER_MFMA_RING_SYNC || inner == SKG_INNER_MFMA_RING_SHARED)
        return mfma_kernel_sync(inner, M, row_tiles, depth);
    if (M > 16) {  // several token tiles of 16
        const int mt = (M + 15) / 16;
        return mt == 2   ? mfma_kernel_mt2(inner, row_tiles, depth)
               : mt == 3 ? mfma_kernel_mt3(inner, row_tiles, depth)
               : mt == 4 ? mfma_kernel_mt4(inner, row_tiles, depth)
                         : nullptr;
    }
    for (int i = 0; i < kNumMfma; ++i) {
        const MfmaVariant &v = kMfmaVariants[i];
        if (v.G != row_tiles || v.PF != depth) continue;
        switch (inner) {
            case SKG_INNER_MFMA: return v.lds_a;
            case SKG_INNER_MFMA_GA: return M <= 8 ? v.ga2 : v.ga4;
            case SKG_INNER_MFMA_RING: return v.ring_lds_a;
            case SKG_INNER_MFMA_RING_GA: return M <= 8 ? v.ring_ga2 : v.ring_ga4;
            default: return nullptr;
        }
    }
    return nullptr;
}

}  // namespace

bool variant_exists(int inner, int row_tiles, int depth, bool f32w, int M) {
    return find_kernel(inner, M, row_tiles, depth, f32w) != nullptr;
}

hipError_t launch(const KParams &p, const Geometry &g, const skg_config &cfg,
                  hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
    KernelPtr fn = find_kernel(cfg.inner, p.M, cfg.row_tiles, cfg.depth, p.w_f32 != 0);
    if (!fn) return hipErrorInvalidValue;
    if (g.lds_bytes > 64 * 1024) {
        // allow this kernel the full LDS of a CU (once per kernel and
        // device: the attribute belongs to the kernel as loaded on one device)
        int dev = 0;
        if (const hipError_t e = hipGetDevice(&dev)) return e;
        static std::mutex mu;
        static std::set<std::pair<int, KernelPtr>> done;
        std::lock_guard<std::mutex> lock(mu);
        if (!done.count(std::make_pair(dev, fn))) {
            // resolving the device function loads the kernel's code object,
            // which the runtime may otherwise defer to the first launch
            // (raising the limit of a kernel whose code object is not loaded
            // fails).  Neither step is fatal: if the limit cannot be raised,
            // the launch below reports whether the LDS it asks for is granted.
            hipFunction_t dev_fn = nullptr;
            (void)hipGetFuncBySymbol(&dev_fn, reinterpret_cast<const void *>(fn));
            if (hipFuncSetAttribute(reinterpret_cast<const void *>(fn),
                                    hipFuncAttributeMaxDynamicSharedMemorySize,
                                    kMaxLdsBytes) == hipSuccess)
                done.insert(std::make_pair(dev, fn));
            (void)hipGetLastError();  // neither failure belongs to the launch
        }
    }
    const unsigned grid = (unsigned)g.grid_rb * (unsigned)cfg.split_k;
    const bool second = p.two_pass != 0;
    const int64_t red_total = (int64_t)p.num_rb * p.M * p.rows_per_wg;
    const unsigned red_grid = (unsigned)std::min<int64_t>((red_total + 255) / 256, 2048);
    if (start || stop) {
        // the dispatches record the kernels' own start (first kernel) and end
        // (last kernel)
        KParams arg = p;
        void *args[] = {&arg};
        hipError_t e = hipExtLaunchKernel(reinterpret_cast<const void *>(fn), dim3(grid),
                                          dim3(g.threads), args, g.lds_bytes, stream, start,
                                          second ? nullptr : stop, 0);
        if (e != hipSuccess || !second) return e;
        return hipExtLaunchKernel(reinterpret_cast<const void *>(skg_splitk_reduce_kernel),
                                  dim3(red_grid), dim3(256), args, 0, stream, nullptr, stop, 0);
    }
    hipLaunchKernelGGL(fn, dim3(grid), dim3(g.threads), g.lds_bytes, stream, p);
    if (second)
        hipLaunchKernelGGL(skg_splitk_reduce_kernel, dim3(red_grid), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_zero_fill(void *C, int M, int N, int64_t ldc, int out_bf16,
                            hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
    const int64_t total = (int64_t)M * N;
    const unsigned blocks = (unsigned)std::min<int64_t>((total + 255) / 256, 4096);
    if (start || stop) {
        void *args[] = {&C, &M, &N, &ldc, &out_bf16};
        return hipExtLaunchKernel(reinterpret_cast<const void *>(skg_zero_fill_kernel),
                                  dim3(blocks), dim3(256), args, 0, stream, start, stop, 0);
    }
    hipLaunchKernelGGL(skg_zero_fill_kernel, dim3(blocks), dim3(256), 0, stream, C, M, N, ldc,
                       out_bf16);
    return hipGetLastError();
}

hipError_t launch_small_k(const KParams &p, hipStream_t stream, hipEvent_t start,
                          hipEvent_t stop) {
    const int64_t total = (int64_t)p.M * p.N;
    const unsigned blocks = (unsigned)std::min<int64_t>((total + 255) / 256, 4096);
    if (start || stop) {
        KParams arg = p;
        void *args[] = {&arg};
        return hipExtLaunchKernel(reinterpret_cast<const void *>(skg_small_k_kernel),
                                  dim3(blocks), dim3(256), args, 0, stream, start, stop, 0);
    }
    hipLaunchKernelGGL(skg_small_k_kernel, dim3(blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_stream_read(const void *src, size_t n16, void *sink, hipStream_t stream) {
    hipLaunchKernelGGL(skg_stream_read_kernel, dim3(kReadProbeGrid), dim3(256), 0, stream,
                       reinterpret_cast<const uint16_t *>(src), n16,
                       reinterpret_cast<unsigned *>(sink));
    return hipGetLastError();
}

hipError_t probe_kernels() {
    hipFuncAttributes attr;
    return hipFuncGetAttributes(&attr, reinterpret_cast<const void *>(skg_zero_fill_kernel));
}

}  // namespace skg

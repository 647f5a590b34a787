// skg_scratch.hip -- the split-K workspace of the no-allocation entry point
// (skinny_gemm_bf16_noalloc): one statically sized array in device memory per
// GPU, created when the code object is loaded, instead of a buffer the
// library allocates per stream.
//
// Layout (32-bit words): kScratchSlotWords words of one-pass split-K tree
// slots (64-bit each), then the fp32 partials of the two-pass split.  The
// slots must be zero when a call starts.  Static storage starts zeroed, the
// first use on a device clears them once more in stream order, and every call
// that completes leaves them at zero (the second workgroup at each tree node
// empties its slot), so no call clears them.  The partials are written before
// they are read within each call.
#include <mutex>

#include "skg_internal.h"

static __device__ __align__(256) unsigned scratch[skg::kScratchWords];

namespace skg {

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_addr[kMaxDevices];  // the array's device address, per device (nullptr: not looked up)

__global__ void skg_clear_words_kernel(unsigned *p, int n) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
        p[i] = 0u;
}

}  // namespace

hipError_t static_scratch(hipStream_t stream, void **ptr) {
    int dev = 0;
    if (const hipError_t e = hipGetDevice(&dev)) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_addr[dev] == nullptr) {
        // the host-side name of the array is not a device address: look the
        // address up once per device, with that device current
        void *addr = nullptr;
        if (const hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch))) return e;
        if (addr == nullptr) return hipErrorInvalidSymbol;
        // a kernel (not a memset), so that a first call under graph capture
        // records nothing a replay could mishandle
        hipLaunchKernelGGL(skg_clear_words_kernel, dim3(256), dim3(256), 0, stream,
                           reinterpret_cast<unsigned *>(addr), kScratchSlotWords);
        if (const hipError_t e = hipGetLastError()) return e;
        g_addr[dev] = addr;
    }
    *ptr = g_addr[dev];
    return hipSuccess;
}

}  // namespace skg

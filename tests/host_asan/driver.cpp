// Host-logic driver run under AddressSanitizer and UndefinedBehaviorSanitizer
// (CPU only, no GPU call is reached): dispatch, configuration checks,
// workspace sizes, warm-up keys, the tier crossover, status strings and every
// argument check, over a grid of shapes and random (also absurd)
// configurations.  Exits non-zero on a wrong answer; the sanitizers abort on
// an out-of-bounds access, a leak or an integer overflow.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "../../include/skinny_gemm.h"

static int failures = 0;
#define EXPECT(cond)                                                        \
    do {                                                                    \
        if (!(cond)) {                                                      \
            std::fprintf(stderr, "FAILED %s at line %d\n", #cond, __LINE__); \
            ++failures;                                                     \
        }                                                                   \
    } while (0)

int main() {
    const int Ks[] = {0, 1, 7, 8, 9, 64, 1000, 1536, 2880, 7168, 14336, 20000, 1 << 20};
    const int Ns[] = {1, 3, 128, 256, 2112, 24576, 1 << 20};
    for (int M = 0; M <= 66; ++M)
        for (int K : Ks)
            for (int N : Ns) {
                skg_config c;
                const int st = skinny_gemm_dispatch(M, K, N, &c);
                if (M < 1) {
                    EXPECT(st == SKG_ERR_INVALID_ARG);
                    continue;
                }
                if (M > SKG_MAX_M) {
                    EXPECT(st == SKG_ERR_UNSUPPORTED);
                    continue;
                }
                // every realistic shape has a configuration; beyond that the
                // answer is UNSUPPORTED, never a configuration that cannot run
                const bool realistic = K <= 20000 && N <= 24576;
                EXPECT(st == SKG_OK || (!realistic && st == SKG_ERR_UNSUPPORTED));
                if (st == SKG_OK) {
                    EXPECT(skinny_gemm_check_config(M, K, N, &c) == SKG_OK);
                    size_t bytes = 0;
                    EXPECT(skinny_gemm_workspace_bytes(M, K, N, &c, &bytes) == SKG_OK);
                    skg_config c2;
                    EXPECT(skinny_gemm_dispatch(M, K, N, &c2) == SKG_OK &&
                           std::memcmp(&c, &c2, sizeof c) == 0);
                }
                skg_config cf;
                const int stf = skinny_gemm_f32w_dispatch(M, K, N, &cf);
                if (M > SKG_MAX_M_VALU) {
                    EXPECT(stf == SKG_ERR_UNSUPPORTED);
                } else {
                    EXPECT(stf == SKG_OK || (!realistic && stf == SKG_ERR_UNSUPPORTED));
                    if (stf == SKG_OK) EXPECT(skinny_gemm_f32w_check_config(M, K, N, &cf) == SKG_OK);
                }
            }
    // random and absurd configurations: the checks answer, never crash
    std::mt19937 rng(7);
    std::uniform_int_distribution<int> any(INT_MIN, INT_MAX);
    std::uniform_int_distribution<int> small(-3, 70);
    for (int i = 0; i < 200000; ++i) {
        skg_config c;
        int32_t *f = &c.backend;
        for (int j = 0; j < 8; ++j) f[j] = (i % 4 == 0) ? any(rng) : small(rng);
        const int M = (i % 3 == 0) ? any(rng) : small(rng);
        const int K = (i % 5 == 0) ? any(rng) : (int)(rng() % 30000);
        const int N = (i % 7 == 0) ? any(rng) : (int)(rng() % 30000) + (i % 2);
        const int st = skinny_gemm_check_config(M, K, N, &c);
        EXPECT(st == SKG_OK || st == SKG_ERR_INVALID_ARG);
        size_t bytes = 0;
        const int sw = skinny_gemm_workspace_bytes(M, K, N, &c, &bytes);
        EXPECT(sw == st);
        EXPECT(skinny_gemm_f32w_check_config(M, K, N, &c) != SKG_OK || st == SKG_OK);
    }
    // warm-up keys: the count, then exactly that many, then fewer
    const int kn[] = {7168, 256, 7168, 384, 2880, 128, 7168, 2112, 1536, 24576, 14336, 7168};
    const int ms[] = {1, 2, 3, 4, 8, 16, 24, 32, 48, 64};
    int n = -1;
    EXPECT(skinny_gemm_warmup_keys(kn, 6, ms, 10, nullptr, 0, &n) == SKG_OK && n > 0);
    std::vector<skg_config> keys(n);
    int n2 = -1;
    EXPECT(skinny_gemm_warmup_keys(kn, 6, ms, 10, keys.data(), n, &n2) == SKG_OK && n2 == n);
    std::vector<skg_config> few(2);
    EXPECT(skinny_gemm_warmup_keys(kn, 6, ms, 10, few.data(), 2, &n2) == SKG_OK && n2 == n);
    EXPECT(std::memcmp(few.data(), keys.data(), 2 * sizeof(skg_config)) == 0);
    EXPECT(skinny_gemm_f32w_warmup_keys(kn, 2, ms, 6, nullptr, 0, &n2) == SKG_OK && n2 > 0);
    EXPECT(skinny_gemm_warmup_keys(kn, -1, ms, 10, nullptr, 0, &n2) == SKG_ERR_INVALID_ARG);
    EXPECT(skinny_gemm_warmup_keys(kn, 6, ms, 10, nullptr, 3, &n2) == SKG_ERR_INVALID_ARG);
    EXPECT(skinny_gemm_warmup_keys(kn, 6, ms, 10, nullptr, 0, nullptr) == SKG_ERR_INVALID_ARG);
    // the crossover
    for (int i = 0; i < 6; ++i) {
        int m = 0;
        EXPECT(skinny_gemm_max_m(kn[2 * i], kn[2 * i + 1], &m) == SKG_OK);
        EXPECT(m >= 1 && m <= SKG_MAX_M);
    }
    int m = 0;
    EXPECT(skinny_gemm_max_m(7168, 0, &m) == SKG_ERR_INVALID_ARG);
    EXPECT(skinny_gemm_max_m(7168, 256, nullptr) == SKG_ERR_INVALID_ARG);
    // status strings
    for (int s = -5; s < 20; ++s) EXPECT(skinny_gemm_strerror(s) != nullptr);
    // argument checks with placeholder pointers: every one returns before any
    // HIP call (M = 0 / N = 0 are no-ops)
    void *P = reinterpret_cast<void *>(uintptr_t(0x100000));
    void *P2 = reinterpret_cast<void *>(uintptr_t(0x100002));
    EXPECT(skinny_gemm_bf16(P, P, P, 65, 256, 7168, 7168, 7168, 256, 0, nullptr) == SKG_ERR_UNSUPPORTED);
    EXPECT(skinny_gemm_bf16(P, P, P, -1, 256, 7168, 7168, 7168, 256, 0, nullptr) == SKG_ERR_INVALID_ARG);
    EXPECT(skinny_gemm_bf16(P, P, P, 4, 256, 7168, 7160, 7168, 256, 0, nullptr) == SKG_ERR_INVALID_ARG);
    EXPECT(skinny_gemm_bf16(P2, P, P, 4, 256, 7168, 7168, 7168, 256, 0, nullptr) == SKG_ERR_MISALIGNED);
    EXPECT(skinny_gemm_bf16(P, P, P, 4, 256, 7168, 7168, 7168, 256, 7, nullptr) == SKG_ERR_INVALID_ARG);
    EXPECT(skinny_gemm_bf16(P, P, P, 0, 256, 7168, 7168, 7168, 256, 0, nullptr) == SKG_OK);
    EXPECT(skinny_gemm_bf16(nullptr, nullptr, nullptr, 4, 0, 7168, 7168, 7168, 0, 0, nullptr) == SKG_OK);
    EXPECT(skinny_gemm_f32w(P, P, P, 17, 256, 7168, 7168, 7168, 256, 0, nullptr) == SKG_ERR_UNSUPPORTED);
    EXPECT(skinny_gemm_f32w(P, P, P, 4, 256, 7168, 7168, 7170, 256, 0, nullptr) == SKG_ERR_MISALIGNED);
    skg_config bad;
    std::memset(&bad, 0, sizeof bad);
    EXPECT(skinny_gemm_bf16_with_config(P, P, P, 4, 256, 7168, 7168, 7168, 256, 0, nullptr, &bad) == SKG_ERR_INVALID_ARG);
    EXPECT(skinny_gemm_bf16_with_config(P, P, P, 4, 256, 7168, 7168, 7168, 256, 0, nullptr, nullptr) == SKG_ERR_INVALID_ARG);
    EXPECT(skinny_gemm_stream_read(P2, 16, P, nullptr) == SKG_ERR_MISALIGNED);
    EXPECT(skinny_gemm_stream_read(nullptr, 16, P, nullptr) == SKG_ERR_INVALID_ARG);
    EXPECT(skinny_gemm_last_hip_error() == 0);
    std::printf("host driver: %d failures\n", failures);
    return failures == 0 ? 0 : 1;
}

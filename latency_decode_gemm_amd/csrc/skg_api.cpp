// skg_api.cpp -- C ABI of the skinny GEMM: argument checks, dispatch,
// launch geometry, per-stream split-K workspace, warm-up.
//
// Dispatch follows the shape-keyed selection on the PR #42562 page
// ("Add generic cuteDSL LL BF16 router (GEMM)", section 实现拆解 item 3 and
// the ll_bf16.py excerpt): a pure function of (M, K, N) that looks up a table
// tuned per (K, N) and M and otherwise falls back to a default.  Here the table
// is compiled in (tuned_table.inc, measured on MI355X) and returns a complete
// skg_config; there is no runtime switch that changes the choice.  The
// warm-up key list keeps the first-seen order of the distinct configurations,
// as get_warmup_keys does on that page.
//
// Eligibility mirrors the router gate of the same page (item 4 and the
// review section 评论区精华): M <= 16 (here 64 with the middle tier of the
// PR #48597 page, section 实现拆解 item 3), bf16 operands, 16-byte aligned 128-bit
// loads; anything else is rejected with a status code so the caller can fall
// back to another GEMM.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <set>
#include <tuple>
#include <utility>
#include <vector>

#include "skg_internal.h"

namespace skg {

namespace {

struct TableEntry {
    int M, K, N;
    skg_config cfg;
};

#include "tuned_table.inc"
#include "tuned_table_f32w.inc"

struct CrossoverEntry {
    int K, N, max_m;
};

#include "crossover_table.inc"

constexpr int kNumTable = sizeof(kTunedTable) / sizeof(kTunedTable[0]);
constexpr int kNumTableF32w = sizeof(kTunedTableF32w) / sizeof(kTunedTableF32w[0]);


// (in 64 bits, so that sizes near the int range cannot overflow)
int ceil_div(int a, int b) { return (int)(((int64_t)a + b - 1) / b); }
int round_up(int a, int b) { return (int)((((int64_t)a + b - 1) / b) * b); }

bool config_equal(const skg_config &a, const skg_config &b) {
    return a.backend == b.backend && a.inner == b.inner && a.split_k == b.split_k &&
           a.row_tiles == b.row_tiles && a.waves_n == b.waves_n && a.waves_k == b.waves_k &&
           a.depth == b.depth && a.rb_per_wg == b.rb_per_wg;
}

// Default for shapes the table does not list: VALU up to M = 8, MFMA above
// (fp32 weights: VALU throughout; above 16 tokens the LDS-ring MFMA kernel,
// depth 2, one K-wave); 4 waves per workgroup (2 on rows x 2 on K); K split
// only when the staged A slice would exceed 64 KB or the row blocks cannot
// cover the 256 CUs; each workgroup then streams enough row blocks to keep
// the grid near 512.
skg_config default_config(int M, int K, int N, bool f32w = false) {
    skg_config c;
    std::memset(&c, 0, sizeof c);
    c.inner = (M > 16 && !f32w)  ? SKG_INNER_MFMA_RING_GA
              : (M > 8 && !f32w) ? SKG_INNER_MFMA_GA
                                 : SKG_INNER_VALU;
    c.row_tiles = (c.inner == SKG_INNER_VALU) ? 2 : 1;
    c.depth = (M > 16) ? 2 : 4;
    c.waves_n = 2;
    c.waves_k = (M > 16) ? 1 : 2;
    const int rows_per_wg = (c.inner == SKG_INNER_VALU ? 4 * c.row_tiles : 16) * c.waves_n;
    const int num_rb = ceil_div(std::max(N, 1), rows_per_wg);
    const int nck = ceil_div(K, kChunk);
    const int step = kValuStep;
    int S = 1;
    while (c.inner == SKG_INNER_VALU && S < 16 &&
           (int64_t)M * ceil_div(nck, S) * kChunk * 2 > 64 * 1024)
        S *= 2;
    while (S < 16 && (int64_t)num_rb * S < 256 && ceil_div(nck, 2 * S) >= 2 * step * c.waves_k)
        S *= 2;
    c.split_k = S;
    c.backend = (S > 1) ? SKG_BACKEND_SPLITK : SKG_BACKEND_DOT;
    c.rb_per_wg = (int)std::max<int64_t>(1, ((int64_t)num_rb * S) / 512);
    Geometry g;
    auto valid = [&](const skg_config &x) {
        return make_geometry(M, K, N, x, &g) &&
               (!f32w || variant_exists(x.inner, x.row_tiles, x.depth, true, M));
    };
    const skg_config first = c;
    // back off until the geometry is valid (an empty last split, LDS size)
    while (c.split_k > 1 && !make_geometry(M, K, N, c, &g)) {
        c.split_k /= 2;
        c.backend = (c.split_k > 1) ? SKG_BACKEND_SPLITK : SKG_BACKEND_DOT;
    }
    while (!make_geometry(M, K, N, c, &g) && c.waves_k > 1) c.waves_k /= 2;
    // the stash holds rb_per_wg row blocks: more workgroups if it does not fit
    while (!make_geometry(M, K, N, c, &g) && c.rb_per_wg > 1) c.rb_per_wg /= 2;
    if (valid(c)) return c;
    // Very long rows or very many of them: keep the split that makes the
    // staged activations fit and give up row blocks per workgroup first,
    // then split K further (one K-wave, one row block as the last resort),
    // then load the activations from global memory instead of staging them.
    skg_config t = first;
    for (t.rb_per_wg = first.rb_per_wg; t.rb_per_wg >= 1; t.rb_per_wg /= 2)
        if (valid(t)) return t;
    for (int S = std::max(2, first.split_k); S <= 4096; S *= 2)
        for (int wk : {first.waves_k, 1})
            for (int rpw : {first.rb_per_wg, 1}) {
                t = first;
                t.split_k = S;
                t.backend = SKG_BACKEND_SPLITK;
                t.waves_k = wk;
                t.rb_per_wg = rpw;
                if (valid(t)) return t;
            }
    t = first;
    t.split_k = 1;
    t.backend = SKG_BACKEND_DOT;
    t.waves_n = 1;
    t.waves_k = 1;
    t.rb_per_wg = 1;
    if (!f32w) {
        t.inner = SKG_INNER_MFMA_GA;
        t.row_tiles = 1;
        t.depth = 2;
    } else {
        t.inner = SKG_INNER_VALU_GA;
        t.row_tiles = 1;
        t.depth = 4;
    }
    if (valid(t)) return t;
    return c;  // nothing runs this shape: the caller reports it
}

// The HIP error behind this thread's last SKG_ERR_HIP (hipSuccess if none).
thread_local int g_last_hip_error = 0;

// SKG_OK if e is hipSuccess, else records e and returns SKG_ERR_HIP.
int hip_status(hipError_t e) {
    if (e == hipSuccess) return SKG_OK;
    g_last_hip_error = (int)e;
    return SKG_ERR_HIP;
}

struct Workspace {
    float *ws = nullptr;  // two-pass partials
    size_t ws_floats = 0;
    unsigned long long *slots = nullptr;  // one-pass tree slots, zero between calls
    size_t slot_words = 0;                // (32-bit words)
};

std::mutex g_ws_mu;
std::map<std::pair<int, void *>, Workspace> g_ws;

// The split-K workspace of (current device, stream), grown if needed.
// Growing is refused while the stream is capturing a graph.  A workspace that
// has been replaced is never freed: a graph captured earlier on this stream
// holds its addresses in its kernel arguments and may be replayed at any time,
// so every buffer stays allocated until the process ends (the sizes only grow,
// so at most a few buffers per stream are ever retired).  The new slots are
// zeroed in stream order before the first kernel that uses them; no host or
// device synchronisation is needed, since no buffer is freed.
int get_workspace(hipStream_t stream, size_t need_floats, size_t need_words, Workspace *out) {
    int dev = 0;
    if (const hipError_t e = hipGetDevice(&dev)) return hip_status(e);
    std::lock_guard<std::mutex> lock(g_ws_mu);
    Workspace &w = g_ws[std::make_pair(dev, (void *)stream)];
    if (w.ws_floats >= need_floats && w.slot_words >= need_words) {
        *out = w;
        return SKG_OK;
    }
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (const hipError_t e = hipStreamIsCapturing(stream, &cap)) return hip_status(e);
    if (cap != hipStreamCaptureStatusNone) return SKG_ERR_NOT_WARMED;
    const size_t nf = std::max(need_floats, w.ws_floats);
    const size_t nw = (std::max(need_words, w.slot_words) + 1) / 2 * 2;  // whole 64-bit slots
    float *ws = nullptr;
    unsigned long long *sl = nullptr;
    if (const hipError_t e = hipMalloc(&ws, std::max<size_t>(nf, 1) * sizeof(float)))
        return hip_status(e);
    if (const hipError_t e = hipMalloc(&sl, std::max<size_t>(nw, 2) * sizeof(unsigned))) {
        (void)hipFree(ws);
        return hip_status(e);
    }
    // (the stream is not capturing here, so this memset is never part of a graph)
    if (const hipError_t e =
            hipMemsetAsync(sl, 0, std::max<size_t>(nw, 2) * sizeof(unsigned), stream)) {
        (void)hipFree(ws);
        (void)hipFree(sl);
        return hip_status(e);
    }
    w.ws = ws;
    w.ws_floats = nf;
    w.slots = sl;
    w.slot_words = nw;
    *out = w;
    return SKG_OK;
}

// Argument checks; f32w: B holds fp32 weights (rows of ldb elements, a
// multiple of 4 so that every row starts 16-byte aligned).
int check_args(const void *A, const void *B, const void *C, int M, int N, int K, int64_t lda,
               int64_t ldb, int64_t ldc, int out_dtype, bool f32w = false) {
    if (M < 0 || N < 0 || K < 0) return SKG_ERR_INVALID_ARG;
    if (M > (f32w ? kMaxMValu : SKG_MAX_M)) return SKG_ERR_UNSUPPORTED;
    if (out_dtype != SKG_OUT_F32 && out_dtype != SKG_OUT_BF16) return SKG_ERR_INVALID_ARG;
    if (M == 0 || N == 0) return SKG_OK;
    if (lda < K || ldb < K || ldc < N) return SKG_ERR_INVALID_ARG;
    if (C == nullptr) return SKG_ERR_INVALID_ARG;
    if (K > 0 && (A == nullptr || B == nullptr)) return SKG_ERR_INVALID_ARG;
    if (K > 0) {
        if ((reinterpret_cast<uintptr_t>(A) & 15u) || (reinterpret_cast<uintptr_t>(B) & 15u))
            return SKG_ERR_MISALIGNED;
        if ((lda & 7) || (ldb & (f32w ? 3 : 7))) return SKG_ERR_MISALIGNED;
    }
    const uintptr_t csz = (out_dtype == SKG_OUT_F32) ? 4u : 2u;
    if (reinterpret_cast<uintptr_t>(C) & (csz - 1)) return SKG_ERR_MISALIGNED;
    return SKG_OK;
}

// Whether cfg's split-K workspace for (M, K, N) fits the static scratch: its
// tree slots in the first kScratchSlotWords words, its partials in the
// kScratchPartialFloats words after them (true without a K split).
bool fits_static_scratch(int M, int K, int N, const skg_config &cfg) {
    if (K < kChunk || cfg.split_k <= 1) return true;  // no workspace
    Geometry g;
    if (!make_geometry(M, K, N, cfg, &g)) return false;
    return g.slot_words <= (size_t)kScratchSlotWords &&
           g.ws_floats <= (size_t)kScratchPartialFloats;
}

// static_ws: the split-K workspace is the per-device static scratch (the
// no-allocation entry point; the caller has checked that it fits) instead
// of the stream's allocated workspace.
int run(const void *A, const void *B, void *C, int M, int N, int K, int64_t lda, int64_t ldb,
        int64_t ldc, int out_dtype, void *stream_v, const skg_config &cfg,
        void *start_v = nullptr, void *stop_v = nullptr, bool f32w = false,
        bool static_ws = false) {
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_v);
    hipEvent_t start = reinterpret_cast<hipEvent_t>(start_v);
    hipEvent_t stop = reinterpret_cast<hipEvent_t>(stop_v);
    if (K == 0) {
        return hip_status(launch_zero_fill(C, M, N, ldc, out_dtype == SKG_OUT_BF16, stream, start,
                                           stop));
    }
    KParams p;
    std::memset(&p, 0, sizeof p);
    p.A = reinterpret_cast<const uint16_t *>(A);
    p.B = reinterpret_cast<const uint16_t *>(B);
    p.C = C;
    p.lda = lda;
    p.ldb = ldb;
    p.ldc = ldc;
    p.M = M;
    p.N = N;
    p.K = K;
    p.out_bf16 = (out_dtype == SKG_OUT_BF16);
    p.w_f32 = f32w ? 1 : 0;
    if (K < kChunk)  // rows shorter than one 16-byte window
        return hip_status(launch_small_k(p, stream, start, stop));
    Geometry g;
    if (!make_geometry(M, K, N, cfg, &g)) return SKG_ERR_INVALID_ARG;
    if (f32w && !variant_exists(cfg.inner, cfg.row_tiles, cfg.depth, true, M))
        return SKG_ERR_INVALID_ARG;
    p.nck = g.nck;
    p.nfull = g.nfull;
    p.split_k = cfg.split_k;
    p.two_pass = (cfg.backend == SKG_BACKEND_SPLITK_2PASS);
    p.even = (cfg.backend == SKG_BACKEND_EVEN);
    p.wg_chunks = g.wg_chunks;
    p.wave_chunks = g.wave_chunks;
    p.waves_n = cfg.waves_n;
    p.waves_k = cfg.waves_k;
    p.rows_per_wg = g.rows_per_wg;
    p.num_rb = g.num_rb;
    p.even_q = g.num_rb > 0 ? N / g.num_rb : 0;
    p.even_r = g.num_rb > 0 ? N % g.num_rb : 0;
    p.grid_rb = g.grid_rb;
    p.lds_stride = g.lds_stride;
    p.stash_offset = g.stash_offset;
    p.tr_offset = g.tr_offset;
    if (cfg.split_k > 1 && static_ws) {
        void *base = nullptr;
        if (const hipError_t e = static_scratch(stream, &base)) return hip_status(e);
        p.slots = reinterpret_cast<unsigned long long *>(base);
        p.ws = reinterpret_cast<float *>(base) + kScratchSlotWords;
    } else if (cfg.split_k > 1) {
        Workspace w;
        const int st = get_workspace(stream, g.ws_floats, g.slot_words, &w);
        if (st != SKG_OK) return st;
        p.ws = w.ws;
        p.slots = w.slots;
    }
    return hip_status(launch(p, g, cfg, stream, start, stop));
}

}  // namespace

bool make_geometry(int M, int K, int N, const skg_config &cfg, Geometry *g) {
    if (M < 1 || M > SKG_MAX_M || K < 0 || N < 1) return false;
    if (K > kMaxK || N > kMaxN) return false;
    if (cfg.backend == SKG_BACKEND_DOT) {
        if (cfg.split_k != 1) return false;
    } else if (cfg.backend == SKG_BACKEND_EVEN) {
        // the 256 x rb_per_wg workgroups are num_rb row blocks x split_k slices
        if (cfg.split_k < 1 || cfg.split_k > 64) return false;
        if (cfg.rb_per_wg < 1 || cfg.rb_per_wg > 64 ||
            (kEvenUnit * cfg.rb_per_wg) % cfg.split_k != 0)
            return false;
    } else if (cfg.backend == SKG_BACKEND_SPLITK || cfg.backend == SKG_BACKEND_SPLITK_2PASS) {
        if (cfg.split_k < 2 || cfg.split_k > 4096) return false;
    } else {
        return false;
    }
    if (cfg.inner < SKG_INNER_VALU || cfg.inner > SKG_INNER_MFMA_RING_SHARED) return false;
    const bool ring = cfg.inner == SKG_INNER_MFMA_RING || cfg.inner == SKG_INNER_MFMA_RING_GA ||
                      cfg.inner == SKG_INNER_MFMA_RING_SYNC ||
                      cfg.inner == SKG_INNER_MFMA_RING_SHARED;
    const bool lds_frag = cfg.inner == SKG_INNER_MFMA || cfg.inner == SKG_INNER_MFMA_RING;
    const bool valu = cfg.inner == SKG_INNER_VALU || cfg.inner == SKG_INNER_VALU_GA;
    // the activation tile of a step shared by the workgroup's waves
    const bool shared_a = cfg.inner == SKG_INNER_MFMA_RING_SHARED;
    // VALU_GA keeps depth x M activation chunks in registers
    if (cfg.inner == SKG_INNER_VALU_GA && (M > 8 || M * cfg.depth > 32)) return false;
    if (valu && M > kMaxMValu) return false;
    if (!variant_exists(cfg.inner, cfg.row_tiles, cfg.depth, false, M)) return false;
    const int mt = (M + 15) / 16;  // MFMA token tiles of 16
    if (cfg.waves_n < 1 || cfg.waves_k < 1 || cfg.waves_n > kMaxWaves ||
        cfg.waves_k > kMaxWaves || cfg.waves_n * cfg.waves_k > kMaxWaves)
        return false;
    if (cfg.rb_per_wg < 1) return false;
    Geometry r;
    r.step = kValuStep;
    r.nck = ceil_div(K, kChunk);
    r.nfull = K / kChunk;
    r.rows_per_wave = valu ? 4 * cfg.row_tiles : 16 * cfg.row_tiles;
    r.rows_per_wg = r.rows_per_wave * cfg.waves_n;
    if (cfg.backend == SKG_BACKEND_EVEN) {
        // rows dealt evenly to 256 x rb_per_wg / split_k row blocks, one
        // workgroup per (row block, K slice)
        if (cfg.rb_per_wg > 64) return false;
        r.num_rb = std::min(N, kEvenUnit * cfg.rb_per_wg / cfg.split_k);
        if (ceil_div(N, r.num_rb) > r.rows_per_wg) return false;
        r.grid_rb = r.num_rb;
    } else {
        r.num_rb = ceil_div(N, r.rows_per_wg);
        r.grid_rb = ceil_div(r.num_rb, cfg.rb_per_wg);
    }
    const int S = cfg.split_k;
    const int per_split = ceil_div(std::max(r.nck, 1), S);
    r.wave_chunks = round_up(ceil_div(per_split, cfg.waves_k), r.step);
    r.wg_chunks = r.wave_chunks * cfg.waves_k;
    if ((int64_t)(S - 1) * r.wg_chunks >= std::max(r.nck, 1)) return false;  // empty split
    // staged activations: VALU rows of lds_stride elements (padded by one
    // chunk); MFMA one 1 KB operand fragment per 32-wide K step; the _GA
    // variants none
    r.lds_stride = r.wg_chunks * kChunk + kChunk;
    size_t a_bytes = 0;
    if (cfg.inner == SKG_INNER_VALU)
        a_bytes = (size_t)M * r.lds_stride * 2;
    else if (lds_frag)
        a_bytes = (size_t)(r.wg_chunks / 4) * 64 * 16 * mt;
    if (a_bytes > (size_t)kMaxLdsBytes) return false;
    r.tr_offset = (int)((a_bytes + 15) / 16 * 16);
    // MFMA: one transpose tile per 16-row tile of B per wave, plus one per
    // token tile for A (GA) (the LDS ring: depth slots of those tiles); with
    // the shared activation ring, the waves' rings hold B only and depth x
    // waves_k activation tiles follow them
    const int tiles = (valu ? 0 : (lds_frag || shared_a) ? cfg.row_tiles : cfg.row_tiles + mt) *
                      (ring ? cfg.depth : 1);
    const size_t tr_bytes = (size_t)cfg.waves_n * cfg.waves_k * tiles * kTileBytes +
                            (shared_a ? (size_t)cfg.depth * cfg.waves_k * mt * kTileBytes : 0);
    r.stash_offset = (int)(r.tr_offset + tr_bytes);
    // stash: every wave's partial sums of each of the workgroup's row blocks
    // (VALU: M x its rows; MFMA: one 16 x 16 fp32 tile per 16 rows and
    // token tile)
    const size_t per_block = valu ? (size_t)M * r.rows_per_wg : (size_t)16 * mt * r.rows_per_wg;
    const size_t blocks_per_wg = (size_t)ceil_div(r.num_rb, r.grid_rb);
    // (a row block covered by one wave is written from registers)
    // (the single-pass split-K combines each output through the stash)
    const bool one_pass = cfg.split_k > 1 && cfg.backend != SKG_BACKEND_SPLITK_2PASS;
    const bool direct = cfg.waves_k == 1 && !one_pass;
    const size_t stash_bytes =
        direct ? 0 : blocks_per_wg * cfg.waves_k * per_block * sizeof(float);
    r.lds_bytes = r.stash_offset + stash_bytes;
    if (r.lds_bytes > (size_t)kMaxLdsBytes) return false;
    r.threads = 64 * cfg.waves_n * cfg.waves_k;
    // two-pass: every slice's partials; one pass: split_k - 1 tree nodes of
    // one 64-bit slot per output
    r.ws_floats = (S > 1 && !one_pass) ? (size_t)r.num_rb * S * M * r.rows_per_wg : 0;
    r.slot_words = one_pass ? (size_t)r.num_rb * (S - 1) * M * r.rows_per_wg * 2 : 0;
    // (the kernels index the slots in 31 bits)
    if (r.slot_words / 2 >= ((size_t)1 << 31)) return false;
    if ((int64_t)r.grid_rb * S > 0x7FFFFFFF) return false;
    *g = r;
    return true;
}

}  // namespace skg

using namespace skg;

namespace {

// Whether cfg can run (M, K, N) over bf16 (f32w false) or fp32 weights.
bool config_ok(int M, int K, int N, const skg_config &cfg, bool f32w) {
    Geometry g;
    if (!make_geometry(M, K, N, cfg, &g)) return false;
    return !f32w || variant_exists(cfg.inner, cfg.row_tiles, cfg.depth, true, M);
}

// The tuned entry for (M, K, N); else, for the same (K, N), the entry of the
// smallest tuned M above M whose configuration can run M (the table is keyed
// by (K, N), then M, and a configuration measured for a few more tokens is
// closer to the best than the default rule); else the default rule.  Pure.
int dispatch_impl(int M, int K, int N, bool f32w, skg_config *out) {
    if (!out) return SKG_ERR_INVALID_ARG;
    const int max_m = f32w ? kMaxMValu : SKG_MAX_M;
    if (M < 1 || K < 0 || N < 1) return M > max_m ? SKG_ERR_UNSUPPORTED : SKG_ERR_INVALID_ARG;
    if (M > max_m) return SKG_ERR_UNSUPPORTED;
    const TableEntry *table = f32w ? kTunedTableF32w : kTunedTable;
    const int n = f32w ? kNumTableF32w : kNumTable;
    const TableEntry *above = nullptr;
    for (int i = 0; i < n; ++i) {
        const TableEntry &e = table[i];
        if (e.K != K || e.N != N || e.M < M || !config_ok(M, K, N, e.cfg, f32w)) continue;
        if (e.M == M) {
            *out = e.cfg;
            return SKG_OK;
        }
        if (!above || e.M < above->M) above = &e;
    }
    if (above) {
        *out = above->cfg;
        return SKG_OK;
    }
    *out = default_config(M, K, N, f32w);
    // (only shapes far outside the decode range, e.g. fp32 weights with
    // millions of columns and more than 8 tokens, have no configuration)
    return config_ok(M, K, N, *out, f32w) ? SKG_OK : SKG_ERR_UNSUPPORTED;
}

// With SKINNY_GEMM_LOG=1 in the environment, the first call of each
// (weights, M, K, N) prints the configuration dispatch chose to stderr.  It
// only reports: nothing in the environment changes what dispatch returns.
void log_choice(bool f32w, int M, int K, int N, const skg_config &c) {
    static const bool on = [] {
        const char *v = std::getenv("SKINNY_GEMM_LOG");
        return v && v[0] == '1';
    }();
    if (!on) return;
    static std::mutex mu;
    static std::set<std::tuple<bool, int, int, int>> seen;
    std::lock_guard<std::mutex> lock(mu);
    if (!seen.insert(std::make_tuple(f32w, M, K, N)).second) return;
    std::fprintf(stderr,
                 "skinny_gemm: %s M=%d K=%d N=%d -> backend %d inner %d split_k %d row_tiles %d "
                 "waves_n %d waves_k %d depth %d rb_per_wg %d\n",
                 f32w ? "fp32 weights" : "bf16", M, K, N, c.backend, c.inner, c.split_k,
                 c.row_tiles, c.waves_n, c.waves_k, c.depth, c.rb_per_wg);
}

// Warm-up keys and warm-up over bf16 (f32w false) or fp32 weights.
int warmup_keys_impl(bool f32w, const int *kn_pairs, int n_shapes, const int *m_values, int n_m,
                     skg_config *out, int capacity, int *n_out) {
    if (n_shapes < 0 || n_m < 0 || capacity < 0 || !n_out) return SKG_ERR_INVALID_ARG;
    if ((n_shapes > 0 && !kn_pairs) || (n_m > 0 && !m_values) || (capacity > 0 && !out))
        return SKG_ERR_INVALID_ARG;
    std::vector<skg_config> keys;
    for (int i = 0; i < n_shapes; ++i) {
        const int K = kn_pairs[2 * i], N = kn_pairs[2 * i + 1];
        for (int j = 0; j < n_m; ++j) {
            skg_config c;
            const int st = dispatch_impl(m_values[j], K, N, f32w, &c);
            if (st != SKG_OK) return st;
            bool seen = false;
            for (const skg_config &k : keys) seen = seen || config_equal(k, c);
            if (!seen) keys.push_back(c);
        }
    }
    for (int i = 0; i < (int)keys.size() && i < capacity; ++i) out[i] = keys[i];
    *n_out = (int)keys.size();
    return SKG_OK;
}

int warmup_impl(bool f32w, const int *kn_pairs, int n_shapes, const int *m_values, int n_m,
                void *stream_v, int *n_configs_out) {
    if (n_shapes < 0 || n_m < 0) return SKG_ERR_INVALID_ARG;
    if ((n_shapes > 0 && !kn_pairs) || (n_m > 0 && !m_values)) return SKG_ERR_INVALID_ARG;
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_v);
    // the distinct configurations, the workspace they need, and a scratch
    // problem large enough to run each of them once
    std::vector<std::pair<skg_config, std::pair<int, int>>> todo;  // cfg, (M, K)
    size_t need_f = 0, need_t = 0, max_a = 0, max_b = 0, max_c = 0;
    for (int i = 0; i < n_shapes; ++i) {
        const int K = kn_pairs[2 * i], N = kn_pairs[2 * i + 1];
        if (K < 0 || N < 1) return SKG_ERR_INVALID_ARG;
        for (int j = 0; j < n_m; ++j) {
            const int M = m_values[j];
            skg_config c;
            const int st = dispatch_impl(M, K, N, f32w, &c);
            if (st != SKG_OK) return st;
            if (K == 0) continue;
            Geometry g;
            if (!make_geometry(M, K, N, c, &g)) return SKG_ERR_INVALID_ARG;
            need_f = std::max(need_f, g.ws_floats);
            need_t = std::max(need_t, g.slot_words);
            bool seen = false;
            for (auto &t : todo)
                seen = seen || (config_equal(t.first, c) && t.second.first == M &&
                                t.second.second == K);
            if (!seen) {
                todo.push_back({c, {M, K}});
                const size_t rows = (size_t)g.rows_per_wg;
                const size_t ld = (size_t)round_up(K, kChunk);
                max_a = std::max(max_a, (size_t)M * ld);
                max_b = std::max(max_b, rows * ld);
                max_c = std::max(max_c, (size_t)M * rows);
            }
        }
    }
    // the no-allocation entry point's scratch address on this device (a
    // lookup and a counter clear, no allocation), so that its first call
    // needs neither
    {
        void *base = nullptr;
        if (const hipError_t e = static_scratch(stream, &base)) return hip_status(e);
    }
    int nd = 0;
    {
        std::vector<skg_config> uniq;
        for (auto &t : todo) {
            bool seen = false;
            for (auto &u : uniq) seen = seen || config_equal(u, t.first);
            if (!seen) uniq.push_back(t.first);
        }
        nd = (int)uniq.size();
    }
    if (n_configs_out) *n_configs_out = nd;
    if (todo.empty()) return SKG_OK;
    if (need_f > 0 || need_t > 0) {
        Workspace w;
        const int st = get_workspace(stream, need_f, need_t, &w);
        if (st != SKG_OK) return st;
    }
    uint16_t *a = nullptr, *b = nullptr;
    float *c = nullptr;
    if (const hipError_t e = hipMalloc(&a, max_a * 2)) return hip_status(e);
    const size_t b_bytes = max_b * (f32w ? 4 : 2);  // weights: bf16 or fp32
    if (const hipError_t e = hipMalloc(&b, b_bytes)) {
        (void)hipFree(a);
        return hip_status(e);
    }
    if (const hipError_t e = hipMalloc(&c, max_c * 4)) {
        (void)hipFree(a);
        (void)hipFree(b);
        return hip_status(e);
    }
    hipError_t e = hipMemsetAsync(a, 0, max_a * 2, stream);
    if (e == hipSuccess) e = hipMemsetAsync(b, 0, b_bytes, stream);
    int rc = hip_status(e);
    for (auto &t : todo) {
        if (rc != SKG_OK) break;
        const int M = t.second.first, K = t.second.second;
        Geometry g;
        make_geometry(M, K, 1, t.first, &g);
        const int ld = round_up(K, kChunk);
        rc = run(a, b, c, M, g.rows_per_wg, K, ld, ld, g.rows_per_wg, SKG_OUT_F32, stream,
                 t.first, nullptr, nullptr, f32w);
    }
    e = hipStreamSynchronize(stream);
    if (e != hipSuccess && rc == SKG_OK) rc = hip_status(e);
    (void)hipFree(a);
    (void)hipFree(b);
    (void)hipFree(c);
    return rc;
}

}  // namespace

extern "C" {

int skinny_gemm_dispatch(int M, int K, int N, skg_config *out) {
    return dispatch_impl(M, K, N, false, out);
}

int skinny_gemm_check_config(int M, int K, int N, const skg_config *cfg) {
    if (!cfg) return SKG_ERR_INVALID_ARG;
    return config_ok(M, K, N, *cfg, false) ? SKG_OK : SKG_ERR_INVALID_ARG;
}

int skinny_gemm_workspace_bytes(int M, int K, int N, const skg_config *cfg, size_t *bytes) {
    if (!cfg || !bytes) return SKG_ERR_INVALID_ARG;
    Geometry g;
    if (!make_geometry(M, K, N, *cfg, &g)) return SKG_ERR_INVALID_ARG;
    *bytes = g.ws_floats * sizeof(float) + g.slot_words * sizeof(unsigned);
    return SKG_OK;
}

int skinny_gemm_bf16(const void *A, const void *B, void *C, int M, int N, int K, int64_t lda,
                     int64_t ldb, int64_t ldc, int out_dtype, void *stream) {
    const int st = check_args(A, B, C, M, N, K, lda, ldb, ldc, out_dtype);
    if (st != SKG_OK || M == 0 || N == 0) return st;
    skg_config cfg;
    const int ds = skinny_gemm_dispatch(M, K, N, &cfg);
    if (ds != SKG_OK) return ds;
    log_choice(false, M, K, N, cfg);
    return run(A, B, C, M, N, K, lda, ldb, ldc, out_dtype, stream, cfg);
}

int skinny_gemm_bf16_noalloc(const void *A, const void *B, void *C, int M, int N, int K,
                             int64_t lda, int64_t ldb, int64_t ldc, int out_dtype, void *stream) {
    const int st = check_args(A, B, C, M, N, K, lda, ldb, ldc, out_dtype);
    if (st != SKG_OK || M == 0 || N == 0) return st;
    skg_config cfg;
    const int ds = skinny_gemm_dispatch(M, K, N, &cfg);
    if (ds != SKG_OK) return ds;
    if (!fits_static_scratch(M, K, N, cfg)) return SKG_ERR_SCRATCH_TOO_SMALL;
    log_choice(false, M, K, N, cfg);
    return run(A, B, C, M, N, K, lda, ldb, ldc, out_dtype, stream, cfg, nullptr, nullptr, false,
               true);
}

int skinny_gemm_bf16_timed(const void *A, const void *B, void *C, int M, int N, int K,
                           int64_t lda, int64_t ldb, int64_t ldc, int out_dtype, void *stream,
                           void *start_event, void *stop_event) {
    const int st = check_args(A, B, C, M, N, K, lda, ldb, ldc, out_dtype);
    if (st != SKG_OK || M == 0 || N == 0) return st;
    skg_config cfg;
    const int ds = skinny_gemm_dispatch(M, K, N, &cfg);
    if (ds != SKG_OK) return ds;
    log_choice(false, M, K, N, cfg);
    return run(A, B, C, M, N, K, lda, ldb, ldc, out_dtype, stream, cfg, start_event, stop_event);
}

int skinny_gemm_bf16_with_config(const void *A, const void *B, void *C, int M, int N, int K,
                                 int64_t lda, int64_t ldb, int64_t ldc, int out_dtype,
                                 void *stream, const skg_config *cfg) {
    if (!cfg) return SKG_ERR_INVALID_ARG;
    const int st = check_args(A, B, C, M, N, K, lda, ldb, ldc, out_dtype);
    if (st != SKG_OK || M == 0 || N == 0) return st;
    Geometry g;
    if (K > 0 && !make_geometry(M, K, N, *cfg, &g)) return SKG_ERR_INVALID_ARG;
    return run(A, B, C, M, N, K, lda, ldb, ldc, out_dtype, stream, *cfg);
}

int skinny_gemm_warmup_keys(const int *kn_pairs, int n_shapes, const int *m_values, int n_m,
                            skg_config *out, int capacity, int *n_out) {
    return warmup_keys_impl(false, kn_pairs, n_shapes, m_values, n_m, out, capacity, n_out);
}

int skinny_gemm_warmup(const int *kn_pairs, int n_shapes, const int *m_values, int n_m,
                       void *stream_v, int *n_configs_out) {
    return warmup_impl(false, kn_pairs, n_shapes, m_values, n_m, stream_v, n_configs_out);
}

// ---- fp32 weights --------------------------------------------------------------

int skinny_gemm_f32w_dispatch(int M, int K, int N, skg_config *out) {
    return dispatch_impl(M, K, N, true, out);
}

int skinny_gemm_f32w_check_config(int M, int K, int N, const skg_config *cfg) {
    if (!cfg) return SKG_ERR_INVALID_ARG;
    return config_ok(M, K, N, *cfg, true) ? SKG_OK : SKG_ERR_INVALID_ARG;
}

int skinny_gemm_f32w_timed(const void *A, const void *W, void *C, int M, int N, int K,
                           int64_t lda, int64_t ldw, int64_t ldc, int out_dtype, void *stream,
                           void *start_event, void *stop_event) {
    const int st = check_args(A, W, C, M, N, K, lda, ldw, ldc, out_dtype, true);
    if (st != SKG_OK || M == 0 || N == 0) return st;
    skg_config cfg;
    const int ds = dispatch_impl(M, K, N, true, &cfg);
    if (ds != SKG_OK) return ds;
    log_choice(true, M, K, N, cfg);
    return run(A, W, C, M, N, K, lda, ldw, ldc, out_dtype, stream, cfg, start_event, stop_event,
               true);
}

int skinny_gemm_f32w(const void *A, const void *W, void *C, int M, int N, int K, int64_t lda,
                     int64_t ldw, int64_t ldc, int out_dtype, void *stream) {
    return skinny_gemm_f32w_timed(A, W, C, M, N, K, lda, ldw, ldc, out_dtype, stream, nullptr,
                                  nullptr);
}

int skinny_gemm_f32w_with_config(const void *A, const void *W, void *C, int M, int N, int K,
                                 int64_t lda, int64_t ldw, int64_t ldc, int out_dtype,
                                 void *stream, const skg_config *cfg) {
    if (!cfg) return SKG_ERR_INVALID_ARG;
    const int st = check_args(A, W, C, M, N, K, lda, ldw, ldc, out_dtype, true);
    if (st != SKG_OK || M == 0 || N == 0) return st;
    if (K > 0 && !config_ok(M, K, N, *cfg, true)) return SKG_ERR_INVALID_ARG;
    return run(A, W, C, M, N, K, lda, ldw, ldc, out_dtype, stream, *cfg, nullptr, nullptr, true);
}

int skinny_gemm_f32w_warmup_keys(const int *kn_pairs, int n_shapes, const int *m_values,
                                 int n_m, skg_config *out, int capacity, int *n_out) {
    return warmup_keys_impl(true, kn_pairs, n_shapes, m_values, n_m, out, capacity, n_out);
}

int skinny_gemm_f32w_warmup(const int *kn_pairs, int n_shapes, const int *m_values, int n_m,
                            void *stream_v, int *n_configs_out) {
    return warmup_impl(true, kn_pairs, n_shapes, m_values, n_m, stream_v, n_configs_out);
}

int skinny_gemm_max_m(int K, int N, int *max_m) {
    if (!max_m || K < 0 || N < 1) return SKG_ERR_INVALID_ARG;
    *max_m = SKG_MAX_M_VALU;
    for (const CrossoverEntry &e : kCrossover)
        if (e.K == K && e.N == N && e.max_m > 0) *max_m = e.max_m;
    return SKG_OK;
}

int skinny_gemm_stream_read(const void *src, size_t bytes, void *sink, void *stream) {
    if (bytes == 0) return SKG_OK;
    if (src == nullptr || sink == nullptr) return SKG_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(src) & 15u) || (bytes & 15u)) return SKG_ERR_MISALIGNED;
    if (reinterpret_cast<uintptr_t>(sink) & 3u) return SKG_ERR_MISALIGNED;
    return hip_status(
        launch_stream_read(src, bytes / 16, sink, reinterpret_cast<hipStream_t>(stream)));
}

int skinny_gemm_last_hip_error(void) { return g_last_hip_error; }

int skinny_gemm_available(void) {
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n < 1) return 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return 0;
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return 0;
    return probe_kernels() == hipSuccess ? 1 : 0;
}

const char *skinny_gemm_strerror(int status) {
    switch (status) {
        case SKG_OK: return "success";
        case SKG_ERR_INVALID_ARG: return "invalid argument";
        case SKG_ERR_UNSUPPORTED: return "unsupported shape (M > 16): use another GEMM";
        case SKG_ERR_MISALIGNED:
            return "misaligned operand: A and B need 16-byte alignment and lda, ldb multiples of 8";
        case SKG_ERR_NOT_WARMED:
            return "stream is capturing and its split-K workspace is too small: warm up first";
        case SKG_ERR_HIP: return "HIP runtime error";
        case SKG_ERR_NO_DEVICE: return "no gfx950 device";
        case SKG_ERR_SCRATCH_TOO_SMALL:
            return "the split-K workspace of this shape exceeds the static scratch of "
                   "skinny_gemm_bf16_noalloc: use skinny_gemm_bf16";
        default: return "unknown status";
    }
}

}  // extern "C"

/*
 * skinny_gemm.h -- C ABI of the MI355X (gfx950) small-M bf16 "skinny" GEMM.
 *
 *     C[m, n] = sum_k A[m, k] * B[n, k]          (C = A . B^T, M <= 64)
 *
 * A (activations, M x K) and B (weights, N x K) are row-major bf16; the sum
 * is accumulated in fp32; C is written as fp32 or as bf16 (round to nearest
 * even), optionally into a strided buffer.
 *
 * Sources on the pages:
 *   - PR #42562 page ("Add generic cuteDSL LL BF16 router (GEMM)"):
 *     section 实现拆解 item 1 (dot-product kernel: one block per row of B,
 *     128-bit loads, shuffle + shared-memory reduction, for small M or
 *     K < 2048), item 2 (split-K kernel: K spread over several blocks whose
 *     partial sums are combined), item 3 (dispatch on M, K, N and a cache of
 *     built kernels, plus a warm-up key list), item 4 (the router gate uses it
 *     only when M <= 16 and the activations are bf16; the review section
 *     评论区精华 adds the weight-dtype guard, the 16-byte alignment of 128-bit
 *     loads and the unsupported non-fp32 output); ll_bf16.py excerpt under
 *     关键源码片段 (dispatch and get_warmup_keys).
 *   - PR #48597 page ("GLM-5.2 Blackwell decode optimizations"), section
 *     实现拆解 item 3 and the key-file list: bf16_skinny_gemm for the qkv_a /
 *     q_b / eh_proj decode projections, with a strided-output test; the same
 *     item chooses among a skinny GEMM for small M, a fused GEMM for middle
 *     M and the library GEMM for large M by measured per-shape thresholds.
 *     Here M <= 16 is the skinny tier and 16 < M <= 64 the middle tier (the
 *     matrix-core kernels with 2 to 4 tiles of 16 tokens);
 *     skinny_gemm_max_m gives the measured crossover to the library GEMM.
 *
 * Conventions shared by every entry point:
 *   - Pointers A, B, C are DEVICE pointers owned by the caller; the library
 *     never frees or retains them beyond the call's stream work.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued asynchronously; no entry point synchronises the host
 *     except skinny_gemm_warmup (which waits for its own launches).
 *   - Strides lda, ldb, ldc are in ELEMENTS.  Element (m, k) of A lives at
 *     A[m*lda + k], (n, k) of B at B[n*ldb + k], (m, n) of C at C[m*ldc + n].
 *     Every other element of the C buffer is left untouched.
 *   - Every function returns an skg_status and never aborts.  Argument
 *     checks run on the host before any HIP call, so an error return leaves
 *     device memory unchanged.
 *   - Thread safety: all entry points may be called from several host
 *     threads.  Calls on different streams use different workspaces; calls
 *     on one stream are ordered by the stream.  (skinny_gemm_bf16_noalloc
 *     is the exception: it uses one workspace per GPU.)
 *   - Split-K workspace: the library allocates one per (device, stream) the
 *     first time a configuration with a K split runs there (or in
 *     skinny_gemm_warmup), grows it when a later call needs more, and never
 *     frees a workspace it has replaced, so a graph captured earlier keeps
 *     valid addresses.  A captured graph uses the workspace of the stream
 *     it was captured on: replaying it while other split-K work on that
 *     workspace runs (calls on the capture stream, or another replay on
 *     another stream) races; replay it on the capture stream.  Growing is
 *     refused during capture (SKG_ERR_NOT_WARMED): warm up first.
 *   - Logging: with SKINNY_GEMM_LOG=1 in the environment, the first GEMM call
 *     of each (weight type, M, K, N) prints the chosen configuration to
 *     stderr.  No environment variable changes the dispatch.
 */
#ifndef SKINNY_GEMM_H
#define SKINNY_GEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SKG_OK = 0,
    SKG_ERR_INVALID_ARG = 1, /* null pointer with non-zero size, negative size,
                                lda < K, ldb < K, ldc < N, bad out_dtype, bad config */
    SKG_ERR_UNSUPPORTED = 2, /* M > 64 (M > 16 over fp32 weights): the caller
                                should use another GEMM */
    SKG_ERR_MISALIGNED = 3,  /* A or B not 16-byte aligned, lda or ldb not a
                                multiple of 8, C not aligned to its element size */
    SKG_ERR_NOT_WARMED = 4,  /* the stream is capturing a graph and its split-K
                                workspace is too small: warm up first */
    SKG_ERR_HIP = 5,         /* a HIP runtime call or a kernel launch failed */
    SKG_ERR_NO_DEVICE = 6,   /* no gfx950 device / the code object does not load */
    SKG_ERR_SCRATCH_TOO_SMALL = 7 /* skinny_gemm_bf16_noalloc only: the shape's
                                     split-K configuration needs more than the
                                     static scratch holds; use skinny_gemm_bf16 */
} skg_status;

typedef enum { SKG_OUT_F32 = 0, SKG_OUT_BF16 = 1 } skg_out_dtype;

typedef enum {
    SKG_BACKEND_DOT = 0,   /* each workgroup covers all of K for its blocks of rows of B */
    SKG_BACKEND_SPLITK = 1, /* split_k workgroups per row block, each one slice of K;
                               the slices' fp32 partials of each output are
                               added pairwise along a fixed binary tree, each
                               value carried by an atomic exchange on the
                               tree node's slot (no fence, no spin-wait); the
                               order of the additions is the tree's, whatever
                               the order in which workgroups finish */
    SKG_BACKEND_SPLITK_2PASS = 2, /* as SPLITK, but a second kernel on the same
                                     stream sums the partials in split order */
    SKG_BACKEND_EVEN = 3 /* 256 * rb_per_wg workgroups (256 CUs: rb_per_wg
                            workgroups per CU) are G = min(N, 256 * rb_per_wg
                            / split_k) row blocks times split_k K slices
                            (split_k >= 1 must divide 256 * rb_per_wg); the N
                            rows are dealt evenly to the G blocks, floor or
                            ceil(N / G) rows each; rows_per_wg (the rows the
                            waves cover) must be at least ceil(N / G).  Lanes
                            past a block's last row re-read that row (the same
                            addresses within one load instruction, so no extra
                            memory traffic) and store nothing.  With split_k
                            >= 2 the slices' fp32 partials are summed as in
                            SKG_BACKEND_SPLITK */
} skg_backend;

typedef enum {
    SKG_INNER_VALU = 0,    /* bf16 dot2 instructions, 16 lanes per row of B;
                              A staged in LDS */
    SKG_INNER_MFMA = 1,    /* 16x16x32 bf16 matrix-core tiles (M padded to a
                              multiple of 16, up to 64);
                              A staged in LDS */
    SKG_INNER_MFMA_GA = 2, /* as SKG_INNER_MFMA, with the activation fragments
                              read from global memory (L2) each K step: no LDS
                              for A, so any K fits in one workgroup */
    SKG_INNER_VALU_GA = 3, /* as SKG_INNER_VALU, with each K step's activation
                              chunks read from global memory (L2) into the
                              load ring: no staging, no LDS for A; M <= 8
                              and M * depth <= 32 */
    SKG_INNER_MFMA_RING = 4,    /* as SKG_INNER_MFMA, with the weight loads
                                   written straight into LDS tiles (a ring of
                                   depth K steps per wave) instead of registers */
    SKG_INNER_MFMA_RING_GA = 5, /* as SKG_INNER_MFMA_GA, with weights and
                                   activation fragments both loaded straight
                                   into the LDS ring */
    SKG_INNER_MFMA_RING_SYNC = 6,   /* as SKG_INNER_MFMA_RING_GA, with the
                                       workgroup's waves meeting at a barrier
                                       every K step; M <= 16, row_tiles 1 or 2 */
    SKG_INNER_MFMA_RING_SHARED = 7  /* as SKG_INNER_MFMA_RING_SYNC, with each K
                                       step's activation tile loaded once per
                                       workgroup (per group of waves on the
                                       same K range) into an LDS ring its waves
                                       share; depth >= 3 */
} skg_inner;

#define SKG_MAX_M 64      /* the matrix-core kinds; the VALU kinds take M <= 16 */
#define SKG_MAX_M_VALU 16
/* Static scratch of skinny_gemm_bf16_noalloc, per GPU: the one-pass split-K
 * tree slots and the two-pass split-K fp32 partials. */
#define SKG_SCRATCH_SLOT_BYTES (1 << 20)
#define SKG_SCRATCH_PARTIAL_BYTES (1 << 20)

/* A kernel configuration: what skinny_gemm_dispatch returns and what
 * skinny_gemm_bf16_with_config accepts.  Plain data; compare field by field. */
typedef struct skg_config {
    int32_t backend;   /* skg_backend; SKG_BACKEND_DOT requires split_k == 1,
                          the split-K backends require split_k >= 2,
                          SKG_BACKEND_EVEN takes either */
    int32_t inner;     /* skg_inner */
    int32_t split_k;   /* workgroups along K per row block */
    int32_t row_tiles; /* rows per wave: VALU 4*row_tiles (1, 2, 4);
                          MFMA and MFMA_GA 16*row_tiles (1, 2, 4) */
    int32_t waves_n;   /* waves per workgroup on different rows */
    int32_t waves_k;   /* waves per workgroup on different K slices of the same
                          rows (combined through LDS); waves_n*waves_k <= 8 */
    int32_t depth;     /* 128-wide K steps of loads kept in flight per wave.
                          Compiled (row_tiles, depth) pairs: VALU (1,4) (1,8)
                          (1,12) (2,2) (2,4) (2,8) (4,2) (4,4); MFMA and MFMA_GA
                          (1,2) (1,3) (1,4) (1,6) (2,1) (2,2) (2,3) (2,4) (4,1)
                          (4,2) */
    int32_t rb_per_wg; /* row blocks (of rows_per_wave*waves_n rows) each workgroup
                          streams one after another, >= 1; sets the grid size */
} skg_config;

/*
 * C = A . B^T with the configuration skinny_gemm_dispatch(M, K, N) returns.
 *   A: device bf16 [M, lda], 16-byte aligned, lda % 8 == 0, lda >= K.
 *   B: device bf16 [N, ldb], 16-byte aligned, ldb % 8 == 0, ldb >= K.
 *   C: device [M, ldc] of fp32 (out_dtype SKG_OUT_F32, 4-byte aligned) or
 *      bf16 (SKG_OUT_BF16, 2-byte aligned, round to nearest even), ldc >= N.
 *   0 <= M <= 64 (M > 64 -> SKG_ERR_UNSUPPORTED), 0 <= N <= 2^30,
 *   0 <= K <= 2^28 (larger: SKG_ERR_INVALID_ARG).
 *   M == 0 or N == 0: nothing is written, SKG_OK.  K == 0: C gets zeros.
 * The result for a given (M, K, N) and inputs is bit-identical from call to
 * call (fixed summation order; no floating-point atomics).
 */
int skinny_gemm_bf16(const void *A, const void *B, void *C, int M, int N, int K,
                     int64_t lda, int64_t ldb, int64_t ldc, int out_dtype,
                     void *stream);

/* Same as skinny_gemm_bf16, and the dispatch of the (single) kernel records
 * start_event when the kernel starts and stop_event when it ends (hipEvent_t
 * handles passed as void*, either may be NULL; created by the caller with
 * timing enabled).  hipEventElapsedTime(start, stop) is then the kernel's own
 * duration, without the launch gap a stream-recorded event pair includes.
 * Nothing is recorded when the call returns early (M == 0 or N == 0, errors). */
int skinny_gemm_bf16_timed(const void *A, const void *B, void *C, int M, int N, int K,
                           int64_t lda, int64_t ldb, int64_t ldc, int out_dtype,
                           void *stream, void *start_event, void *stop_event);

/*
 * Same as skinny_gemm_bf16 (same arguments, configuration, kernels and bits),
 * for callers that cannot allocate device memory: code under HIP graph
 * capture without a prior warm-up, tight serving loops, harnesses that forbid
 * allocation.  It calls no hipMalloc, hipFree or other allocating routine.
 * The split-K workspace is one statically sized array per GPU in the
 * library's code object, not a per-stream buffer:
 *   - SKG_SCRATCH_SLOT_BYTES of one-pass split-K tree slots and
 *     SKG_SCRATCH_PARTIAL_BYTES of two-pass fp32 partials (2 MiB per GPU the
 *     library runs on, held until the process ends).  That covers every
 *     configuration dispatch returns for M <= 16 (the largest needs
 *     144 KB) and the middle tier except its two-pass configurations on
 *     wide N (e.g. M > 32 at K = 7168, N = 2112).  A shape whose
 *     configuration needs more returns SKG_ERR_SCRATCH_TOO_SMALL before any
 *     GPU work.
 *   - Every call on one GPU shares that GPU's array.  Calls that overlap in
 *     time on one GPU (on different streams, or a graph replayed beside
 *     them) RACE on it and may return wrong results: serialise them, e.g. on
 *     one stream.  Calls whose configuration has no K split (most large
 *     shapes) do not touch the array.
 *   - The slots must be zero when a call starts: they start at zero, the
 *     first call on a device clears them in stream order (a kernel, not a
 *     memset), and every call that completes leaves them at zero.
 *   - The first call on a device looks up the array's address (per device,
 *     with that device current); skinny_gemm_warmup does the same lookup, so
 *     calling it beforehand keeps that step out of a later capture.
 */
int skinny_gemm_bf16_noalloc(const void *A, const void *B, void *C, int M, int N, int K,
                             int64_t lda, int64_t ldb, int64_t ldc, int out_dtype,
                             void *stream);

/* Same as skinny_gemm_bf16 with an explicit configuration (tests, tuning).
 * An invalid or unsupported configuration returns SKG_ERR_INVALID_ARG. */
int skinny_gemm_bf16_with_config(const void *A, const void *B, void *C, int M,
                                 int N, int K, int64_t lda, int64_t ldb,
                                 int64_t ldc, int out_dtype, void *stream,
                                 const skg_config *cfg);

/* The configuration used for (M, K, N).  Pure host function: no GPU access,
 * deterministic, the same answer on every call.  M must be in 1..64,
 * K >= 0, N >= 1; otherwise SKG_ERR_INVALID_ARG / SKG_ERR_UNSUPPORTED.
 * SKG_ERR_UNSUPPORTED also when no configuration can run the shape (only far
 * outside the decode range).  The returned configuration always passes
 * skinny_gemm_check_config. */
int skinny_gemm_dispatch(int M, int K, int N, skg_config *out);

/* Whether cfg can run (M, K, N): SKG_OK or SKG_ERR_INVALID_ARG.  Pure host. */
int skinny_gemm_check_config(int M, int K, int N, const skg_config *cfg);

/* Bytes of split-K workspace cfg needs for (M, K, N): the tree slots of the
 * one-pass split (SKG_BACKEND_SPLITK, and SKG_BACKEND_EVEN with split_k >= 2:
 * 8 bytes per output and tree node, split_k - 1 nodes) or the partials of the
 * two-pass split (4 bytes per output and slice); 0 without a K split.  Pure
 * host. */
int skinny_gemm_workspace_bytes(int M, int K, int N, const skg_config *cfg,
                                size_t *bytes);

/*
 * Warm-up keys: the distinct results of skinny_gemm_dispatch(M, K, N) for
 * every (K, N) in kn_pairs (n_shapes pairs, laid out K0, N0, K1, N1, ...) and
 * every M in m_values, in first-seen order (shapes outer, M inner).  Writes at
 * most `capacity` configs to `out` (may be NULL when capacity is 0) and the
 * total count to *n_out.  Pure host.
 */
int skinny_gemm_warmup_keys(const int *kn_pairs, int n_shapes,
                            const int *m_values, int n_m, skg_config *out,
                            int capacity, int *n_out);

/*
 * Prepares `stream` for every (K, N) x M combination: makes sure the code
 * object is loaded, sizes this stream's split-K workspace for the largest
 * combination, and runs each distinct configuration once on a small scratch
 * problem.  Idempotent.  Allocates device memory and synchronises `stream`;
 * call it before graph capture.  *n_configs_out (may be NULL) receives the
 * number of distinct configurations.
 */
int skinny_gemm_warmup(const int *kn_pairs, int n_shapes, const int *m_values,
                       int n_m, void *stream, int *n_configs_out);

/*
 * The router GEMM over fp32 weights: C[m, n] = sum_k A[m, k] * W[n, k] with
 * A bf16 and W fp32 (each product one fp32 fused multiply-add of the widened
 * activation, fp32 accumulation).  The PR #48597 page ("GLM-5.2 Blackwell
 * decode optimizations", section 关联脉络) names a router GEMM over fp32
 * weights, and the keeping of router weights in fp32, among that PR's parts;
 * the PR #42562 page (section 风险与影响) notes that its bf16 kernel leaves
 * fp32 weights to other paths.  Same conventions as the bf16 entry points,
 * except:
 *   W: device fp32 [N, ldw], 16-byte aligned, ldw % 4 == 0, ldw >= K
 *      (else SKG_ERR_MISALIGNED / SKG_ERR_INVALID_ARG).
 * Only the VALU inner products (SKG_INNER_VALU, SKG_INNER_VALU_GA) take fp32
 * weights; every backend does.  The configurations come from a table of
 * their own (skinny_gemm_f32w_dispatch).
 */
int skinny_gemm_f32w(const void *A, const void *W, void *C, int M, int N, int K,
                     int64_t lda, int64_t ldw, int64_t ldc, int out_dtype, void *stream);

/* skinny_gemm_f32w with kernel start/end recorded into caller events, as
 * skinny_gemm_bf16_timed does. */
int skinny_gemm_f32w_timed(const void *A, const void *W, void *C, int M, int N, int K,
                           int64_t lda, int64_t ldw, int64_t ldc, int out_dtype,
                           void *stream, void *start_event, void *stop_event);

/* skinny_gemm_f32w with an explicit configuration (tests, tuning); a
 * configuration that cannot run over fp32 weights returns SKG_ERR_INVALID_ARG. */
int skinny_gemm_f32w_with_config(const void *A, const void *W, void *C, int M,
                                 int N, int K, int64_t lda, int64_t ldw,
                                 int64_t ldc, int out_dtype, void *stream,
                                 const skg_config *cfg);

/* The configuration skinny_gemm_f32w uses for (M, K, N); pure host, as
 * skinny_gemm_dispatch. */
int skinny_gemm_f32w_dispatch(int M, int K, int N, skg_config *out);

/* Whether cfg can run (M, K, N) over fp32 weights; pure host. */
int skinny_gemm_f32w_check_config(int M, int K, int N, const skg_config *cfg);

/* Warm-up keys and warm-up for fp32 weights, as skinny_gemm_warmup_keys and
 * skinny_gemm_warmup (the same arguments and behaviour, over
 * skinny_gemm_f32w_dispatch). */
int skinny_gemm_f32w_warmup_keys(const int *kn_pairs, int n_shapes,
                                 const int *m_values, int n_m, skg_config *out,
                                 int capacity, int *n_out);
int skinny_gemm_f32w_warmup(const int *kn_pairs, int n_shapes, const int *m_values,
                            int n_m, void *stream, int *n_configs_out);

/* The hipError_t value behind this thread's most recent SKG_ERR_HIP from a
 * GEMM call, zero-fill or streaming read (0 if there was none): a launch
 * failure reports the runtime's own code here. */
int skinny_gemm_last_hip_error(void);

/* 1 if a gfx950 device is current and the library's kernels load, else 0.
 * The counterpart of is_available in the ll_bf16.py excerpt of the PR #42562
 * page (section 关键源码片段), which tells the router gate whether the
 * kernel path can run on the current device before it is chosen. */
int skinny_gemm_available(void);

/* Measurement aid, not part of the GEMM: streams `bytes` bytes from the
   device buffer `src` with the GEMM's own load form (128-bit non-temporal
   loads; 512 workgroups of 256 threads, 8 loads per thread in flight per
   round) and folds them (XOR of 32-bit words) into `sink`, one 32-bit word
   per workgroup (device memory, at least 2048 bytes, caller-owned).  The XOR
   of the 512 words equals the XOR of all 32-bit words of the buffer.  The
   duration of this kernel is the streaming-read ceiling the GEMM's
   bandwidth figures are compared with.  `src` 16-byte aligned and `bytes` a
   multiple of 16 (else SKG_ERR_MISALIGNED); bytes == 0 is a no-op. */
int skinny_gemm_stream_read(const void *src, size_t bytes, void *sink, void *stream);

/*
 * The measured crossover of the tiers for (K, N): *max_m receives the largest
 * M for which this library was measured faster than the library GEMM
 * (hipBLASLt through torch.nn.functional.linear, both timed as back-to-back
 * calls from a HIP graph over weight copies rotated past the Infinity Cache)
 * at every measured M up to it; a caller uses skinny_gemm_bf16 for
 * M <= *max_m and the library GEMM above.  Shapes that were not measured get
 * SKG_MAX_M_VALU.  Pure host.  (The pages' skinny_max threshold per (N, K),
 * PR #48597 page, section 实现拆解 item 3.)
 */
int skinny_gemm_max_m(int K, int N, int *max_m);

/* Static description of a status code. */
const char *skinny_gemm_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* SKINNY_GEMM_H */

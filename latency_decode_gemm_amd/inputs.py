"""Seeded synthetic inputs for the skinny GEMM (shared by tests, bench, smoke).

This module holds no arithmetic of the GEMM itself: it only draws the
activations A[M, K] and weights B[N, K] and stores them as bf16 bit patterns
(numpy ``uint16``), which both the HIP path and the CPU oracle take as input.

Recipe (the decode workloads on the pages: MoE router gate with 256/384
experts x hidden 7168, a ragged K = 2880, and bf16 qkv_a / q_b / eh_proj
projections; PR #42562 page section 功能与动机 and 实现拆解 item 6, PR #48597
page section 实现拆解 item 3):

* z ~ N(0, 1), drawn as float32 by ``numpy.random.Generator(PCG64(seed))
  .standard_normal(dtype=float32)`` in row-major order;
* A[m, k] = bf16(z),  B[n, k] = bf16(z / sqrt(K))  (unit-variance dot products);
* bf16() is float32 -> bf16 round-to-nearest-even of the bit pattern;
* seeds: seed_A = 1_000_003*K + 10_007*N + M,
         seed_B(r) = 7_919*K + 104_729*N + r  (r = copy index).

Padding columns of a padded leading dimension (lda > K or ldb > K) are
filled with a quiet-NaN bf16 pattern, so any read of them by a kernel shows
up as a NaN in the result.
"""
from __future__ import annotations

import numpy as np

PAD_BITS = np.uint16(0x7FC1)  # quiet NaN, distinctive payload


def seed_a(M: int, K: int, N: int) -> int:
    return 1_000_003 * K + 10_007 * N + M


def seed_b(K: int, N: int, r: int = 0) -> int:
    return 7_919 * K + 104_729 * N + r


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (NaN -> 0x7FC0)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    r = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = np.uint16(0x7FC0) | ((u[nan] >> np.uint32(16)) & np.uint32(0x8000)).astype(np.uint16)
    return r


def _normal_bits(rows: int, K: int, ld: int, seed: int, scale: float) -> np.ndarray:
    gen = np.random.Generator(np.random.PCG64(seed))
    out = np.full((rows, ld), PAD_BITS, dtype=np.uint16)
    if rows == 0 or K == 0:
        return out
    # draw in row blocks to bound the float32 temporaries for huge B
    step = max(1, (1 << 24) // max(K, 1))
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        z = gen.standard_normal((r1 - r0, K), dtype=np.float32)
        if scale != 1.0:
            z *= np.float32(scale)
        out[r0:r1, :K] = f32_to_bf16_bits(z)
    return out


def make_a(M: int, K: int, N: int, lda: int | None = None, seed: int | None = None) -> np.ndarray:
    """Activations A[M, lda] (bf16 bits), values ~ N(0, 1) in the first K columns."""
    lda = K if lda is None else lda
    return _normal_bits(M, K, lda, seed_a(M, K, N) if seed is None else seed, 1.0)


def make_b(K: int, N: int, ldb: int | None = None, r: int = 0, seed: int | None = None) -> np.ndarray:
    """Weights B[N, ldb] (bf16 bits), values ~ N(0, 1/K) in the first K columns."""
    ldb = K if ldb is None else ldb
    scale = 1.0 / np.sqrt(K) if K > 0 else 1.0
    return _normal_bits(N, K, ldb, seed_b(K, N, r) if seed is None else seed, float(scale))


PAD_F32 = np.uint32(0x7FC00001)  # quiet NaN, distinctive payload


def make_w_f32(K: int, N: int, ldw: int | None = None, r: int = 0,
               seed: int | None = None) -> np.ndarray:
    """fp32 weights W[N, ldw] for the fp32-weight router GEMM: the same draws
    z / sqrt(K) as make_b (same seed), kept in float32 instead of being
    rounded to bf16; padding columns hold a quiet NaN."""
    ldw = K if ldw is None else ldw
    out = np.full((N, ldw), PAD_F32, dtype=np.uint32).view(np.float32)
    if N == 0 or K == 0:
        return out
    gen = np.random.Generator(np.random.PCG64(seed_b(K, N, r) if seed is None else seed))
    scale = np.float32(1.0 / np.sqrt(K))
    step = max(1, (1 << 24) // K)
    for r0 in range(0, N, step):
        r1 = min(N, r0 + step)
        z = gen.standard_normal((r1 - r0, K), dtype=np.float32)
        z *= scale
        out[r0:r1, :K] = z
    return out


def make_inputs(M: int, K: int, N: int, lda: int | None = None, ldb: int | None = None,
                r: int = 0):
    """(A_bits [M, lda], B_bits [N, ldb]) for one workload point."""
    return make_a(M, K, N, lda), make_b(K, N, ldb, r)


# The five workload groups (29 distinct (M, K, N) points).
#   out: "f32" or "bf16"; ldc: None means ldc = N.
WORKLOADS = {
    "router_single": [dict(M=1, K=7168, N=256, out="f32", ldc=None)],
    "router_sweep": [dict(M=m, K=7168, N=n, out="f32", ldc=None)
                     for n in (256, 384) for m in (1, 2, 3, 4, 8, 16)],
    "ragged_k2880": [dict(M=m, K=2880, N=128, out="f32", ldc=None) for m in (1, 4, 16)],
    "qkv_a_strided": [dict(M=m, K=7168, N=2112, out="bf16", ldc=4096) for m in (2, 3, 8, 16)],
    "wide_deep": [dict(M=m, K=k, N=n, out="bf16", ldc=None)
                  for (k, n) in ((1536, 24576), (14336, 7168)) for m in (1, 2, 4, 8, 16)],
}


# The router GEMM over fp32 weights (bf16 activations, fp32 output): the
# router sweep's shapes.
WORKLOADS_F32W = {
    "router_f32w": [dict(M=m, K=7168, N=n, out="f32", ldc=None, w="f32")
                    for n in (256, 384) for m in (1, 2, 3, 4, 8, 16)],
}


# The middle tier (16 < M <= 64) on the projection shapes: qkv_a-style into
# the strided bf16 buffer, the wide and the deep projection.
WORKLOADS_MID = {
    "mid_m": [dict(M=m, K=k, N=n, out="bf16", ldc=ldc)
              for (k, n, ldc) in ((7168, 2112, 4096), (1536, 24576, None), (14336, 7168, None))
              for m in (24, 32, 48, 64)],
    # the router and ragged-K shapes beyond 16 tokens (fp32 out), where the
    # crossover to the library GEMM is measured too
    "mid_router": [dict(M=m, K=k, N=n, out="f32", ldc=None)
                   for (k, n) in ((7168, 256), (7168, 384), (2880, 128))
                   for m in (24, 32, 48, 64)],
}


# One decode layer's chain of GEMMs at a small batch (the analogue of the
# launch-latency hiding the pages pursue with programmatic dependent launch):
# the MoE router over fp32 weights, the qkv_a-style projection into its
# strided buffer, the wide and the deep projection, back to back.
WORKLOADS_CHAIN = {
    "decode_chain": [dict(M=4, K=7168, N=256, out="f32", ldc=None, w="f32"),
                     dict(M=4, K=7168, N=2112, out="bf16", ldc=4096),
                     dict(M=4, K=1536, N=24576, out="bf16", ldc=None),
                     dict(M=4, K=14336, N=7168, out="bf16", ldc=None)],
}


def all_points():
    """Distinct (M, K, N, out, ldc) points over all workload groups, first-seen order."""
    seen, pts = set(), []
    for group in WORKLOADS.values():
        for p in group:
            key = (p["M"], p["K"], p["N"], p["out"], p["ldc"])
            if key not in seen:
                seen.add(key)
                pts.append(dict(p))
    return pts

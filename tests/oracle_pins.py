"""Pins for the CPU oracle: checks that hold for the true C = A . B^T.

Each ``pin_*`` takes a GEMM function ``gemm(A_bits, B_bits, K) -> float64[M, N]``
(A_bits [M, lda], B_bits [N, ldb], uint16 bf16 patterns) and returns a list of
failure messages (empty = pass).  They are run against the oracle (must all
pass) and against oracles with a planted mistake (each must fail at least one),
so a plausible slip anywhere in the oracle -- a dropped term, a wrong index or
stride, a transposed operand, a wrong sign, a wrong decode, a low-precision
sum -- is caught by something other than the oracle itself.

Nothing here calls the HIP library.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

from latency_decode_gemm_amd.inputs import f32_to_bf16_bits

ONE = np.uint16(0x3F80)


def _dec(bits) -> np.ndarray:
    # independent decode for the pins: exponent/fraction arithmetic, no bit cast
    b = np.asarray(bits, dtype=np.int64)
    s = np.where((b >> 15) & 1, -1.0, 1.0)
    e = (b >> 7) & 0xFF
    f = (b & 0x7F).astype(np.float64)
    val = np.where(e == 0, f / 128.0 * 2.0 ** -126, (1.0 + f / 128.0) * np.exp2(e.astype(np.float64) - 127.0))
    return s * val


def _rand_bits(rng, shape, scale=1.0):
    return f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


def pin_one_hot(gemm) -> list:
    """A[m, :] = e_{k_m}  =>  C[m, n] == B[n, k_m] exactly.  The k_m cover the
    first and last column, chunk borders and the ragged K = 2880 end."""
    fails = []
    rng = np.random.default_rng(11)
    for K, ks in ((2880, (0, 7, 8, 2047, 2048, 2559, 2560, 2873, 2879)),
                  (37, (0, 1, 8, 31, 32, 36)), (9, (0, 8))):
        M = len(ks)
        N = 19
        A = np.zeros((M, K), dtype=np.uint16)
        for m, k in enumerate(ks):
            A[m, k] = ONE
        B = _rand_bits(rng, (N, K))
        C = np.asarray(gemm(A, B, K))
        want = _dec(B[:, list(ks)]).T
        if C.shape != want.shape or not np.array_equal(C, want):
            fails.append(f"one-hot K={K}")
    return fails


def pin_identity(gemm) -> list:
    """N = K and B = I  =>  C == A exactly."""
    fails = []
    rng = np.random.default_rng(12)
    for K, M in ((16, 16), (128, 5), (2880, 3)):
        A = _rand_bits(rng, (M, K))
        B = np.zeros((K, K), dtype=np.uint16)
        B[np.arange(K), np.arange(K)] = ONE
        C = np.asarray(gemm(A, B, K))
        if not np.array_equal(C, _dec(A)):
            fails.append(f"identity K={K}")
    return fails


def pin_constant(gemm) -> list:
    """A = a, B = b everywhere  =>  C == K*a*b (values chosen bf16-exact)."""
    fails = []
    cases = [  # (K, a_bits, b_bits, expected)
        (7168, 0x3F80, 0x3C80, 112.0),      # 1 * 2^-6
        (2880, 0x3F80, 0x3C80, 45.0),
        (1536, 0x3F80, 0x3C80, 24.0),
        (14336, 0x3F80, 0x3C80, 224.0),
        (7168, 0xBFC0, 0x3F40, -8064.0),    # -1.5 * 0.75
        (3, 0x4040, 0xC000, -18.0),         # 3 * -2
    ]
    for K, ab, bb, want in cases:
        A = np.full((2, K), ab, dtype=np.uint16)
        B = np.full((3, K), bb, dtype=np.uint16)
        C = np.asarray(gemm(A, B, K))
        if C.shape != (2, 3) or not np.all(C == want):
            fails.append(f"constant K={K} want {want}")
    return fails


def pin_bruteforce(gemm, n_cases: int = 50) -> list:
    """Tiny random shapes against exact rational sums: the binary64 result of a
    k-ordered sum of exact products differs from the exact value by at most
    gamma_{K-1} * sum_k |a_k b_k| with gamma_n = n u / (1 - n u), u = 2^-53."""
    fails = []
    rng = np.random.default_rng(13)
    u = 2.0 ** -53
    Ks = list(range(1, 41)) + [511, 512, 513, 1023, 1024, 1025, 2047, 2048, 2049, 2880]
    for i in range(n_cases):
        M = int(rng.integers(1, 17))
        N = int(rng.integers(1, 34))
        K = int(Ks[i % len(Ks)]) if i < len(Ks) else int(rng.integers(1, 41))
        if K > 600:
            M, N = min(M, 2), min(N, 3)
        A = _rand_bits(rng, (M, K))
        B = _rand_bits(rng, (N, K), 1.0 / math.sqrt(K))
        C = np.asarray(gemm(A, B, K))
        if C.shape != (M, N):
            fails.append(f"bruteforce shape {C.shape} != {(M, N)}")
            continue
        Ad, Bd = _dec(A), _dec(B)
        gam = (K - 1) * u / (1 - (K - 1) * u) if K > 1 else 0.0
        for m in range(M):
            for n in range(N):
                exact = sum((Fraction(float(x)) * Fraction(float(y)) for x, y in zip(Ad[m], Bd[n])),
                            Fraction(0))
                bound = gam * float(np.sum(np.abs(Ad[m] * Bd[n])))
                if abs(Fraction(float(C[m, n])) - exact) > Fraction(bound):
                    fails.append(f"bruteforce M={M} N={N} K={K} at ({m},{n})")
                    break
            else:
                continue
            break
    return fails


def pin_numpy(gemm) -> list:
    """Against numpy's binary64 matmul of the decoded inputs (a textbook
    library routine): normalised difference <= 1e-12."""
    fails = []
    rng = np.random.default_rng(14)
    for (M, N, K) in ((16, 33, 2880), (3, 64, 7168), (1, 5, 1), (7, 9, 1537)):
        A = _rand_bits(rng, (M, K))
        B = _rand_bits(rng, (N, K), 1.0 / math.sqrt(K))
        C = np.asarray(gemm(A, B, K))
        Ad, Bd = _dec(A), _dec(B)
        R = Ad @ Bd.T
        den = np.outer(np.linalg.norm(Ad, axis=1), np.linalg.norm(Bd, axis=1))
        if C.shape != R.shape or np.max(np.abs(C - R) / den) > 1e-12:
            fails.append(f"numpy M={M} N={N} K={K}")
    return fails


def pin_invariants(gemm) -> list:
    """Permuting B's rows permutes C's columns; a row of C depends only on the
    same row of A; scaling A by 2^j scales C by 2^j; splitting K adds up."""
    fails = []
    rng = np.random.default_rng(15)
    M, N, K = 5, 23, 300
    A = _rand_bits(rng, (M, K))
    B = _rand_bits(rng, (N, K), 0.1)
    C = np.asarray(gemm(A, B, K))
    perm = rng.permutation(N)
    if not np.array_equal(np.asarray(gemm(A, B[perm], K)), C[:, perm]):
        fails.append("row permutation")
    A2 = A.copy()
    A2[2] = _rand_bits(rng, (1, K))[0]
    C2 = np.asarray(gemm(A2, B, K))
    if not np.array_equal(np.delete(C2, 2, axis=0), np.delete(C, 2, axis=0)):
        fails.append("row independence")
    # A * 4: add 2 to the biased exponent of every normal, non-zero value
    A4 = A.copy().astype(np.int64)
    nz = (A4 & 0x7F80) != 0
    A4[nz] += 2 << 7
    C4 = np.asarray(gemm(A4.astype(np.uint16), B, K))
    if not np.array_equal(C4, 4.0 * C):
        fails.append("power-of-two scaling")
    K1 = 123
    Ca = np.asarray(gemm(np.ascontiguousarray(A[:, :K1]), np.ascontiguousarray(B[:, :K1]), K1))
    Cb = np.asarray(gemm(np.ascontiguousarray(A[:, K1:]), np.ascontiguousarray(B[:, K1:]), K - K1))
    den = np.outer(np.linalg.norm(_dec(A), axis=1), np.linalg.norm(_dec(B), axis=1))
    if np.max(np.abs(Ca + Cb - C) / den) > 1e-13:
        fails.append("K-split additivity")
    return fails


def pin_padding(gemm) -> list:
    """A padded leading dimension (NaN in the padding) changes nothing."""
    fails = []
    rng = np.random.default_rng(16)
    M, N, K = 4, 9, 45
    A = _rand_bits(rng, (M, K))
    B = _rand_bits(rng, (N, K))
    Ap = np.full((M, 56), 0x7FC1, dtype=np.uint16)
    Bp = np.full((N, 64), 0x7FC1, dtype=np.uint16)
    Ap[:, :K] = A
    Bp[:, :K] = B
    C = np.asarray(gemm(A, B, K))
    Cp = np.asarray(gemm(Ap, Bp, K))
    if not np.array_equal(C, Cp):
        fails.append("padded leading dimension")
    return fails


def pin_degenerate(gemm) -> list:
    """K = 0 gives zeros of shape [M, N]; M = 0 or N = 0 gives an empty result."""
    fails = []
    A = np.zeros((3, 8), dtype=np.uint16)
    B = np.full((4, 8), 0x3F80, dtype=np.uint16)
    C = np.asarray(gemm(A, B, 0))
    if C.shape != (3, 4) or np.any(C != 0):
        fails.append("K=0")
    if np.asarray(gemm(np.zeros((0, 8), np.uint16), B, 8)).size != 0:
        fails.append("M=0")
    if np.asarray(gemm(A, np.zeros((0, 8), np.uint16), 8)).size != 0:
        fails.append("N=0")
    return fails


ALL_PINS = [pin_one_hot, pin_identity, pin_constant, pin_bruteforce, pin_numpy,
            pin_invariants, pin_padding, pin_degenerate]


def run_all(gemm) -> list:
    fails = []
    for p in ALL_PINS:
        try:
            fails += p(gemm)
        except Exception as e:  # a mutant may also crash a pin
            fails.append(f"{p.__name__} raised {type(e).__name__}: {e}")
    return fails

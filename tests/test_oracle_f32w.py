"""The fp32-weight oracle (C = A . W^T, A bf16, W binary32) against what the
mathematics fixes, and planted mistakes that those pins must catch (CPU only).

The pins:
* one-hot activation rows select weights exactly (C[m, n] = W[n, k_m], for
  weights with all 24 significant bits in use, so any rounding of W shows);
* weights that are bf16 values reduce it to the bf16 oracle, bit for bit;
* constant inputs give the closed form K * a * w exactly;
* exact rational sums on tiny random shapes, within the binary64 bound;
* numpy's binary64 matmul on decoded inputs (<= 1e-12 normalised);
* NaN padding beyond K never leaks in; degenerate sizes.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle

ONE = np.uint16(0x3F80)    # bf16 1.0
M1P5 = np.uint16(0xBFC0)   # bf16 -1.5


def _rand_a(rng, shape):
    z = rng.standard_normal(shape).astype(np.float32)
    u = z.view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _rand_w(rng, shape, scale=1.0):
    return (rng.standard_normal(shape) * scale).astype(np.float32)


def pin_one_hot(gemm):
    bad = []
    rng = np.random.default_rng(10)
    for K in (1, 8, 9, 2880, 7168):
        N = 19
        W = _rand_w(rng, (N, K))
        ks = sorted({0, K - 1, K // 2, min(K - 1, 2047), min(K - 1, 2559)})
        A = np.zeros((len(ks), K), np.uint16)
        for m, k in enumerate(ks):
            A[m, k] = ONE
        C = gemm(A, W, K)
        want = W[:, ks].T.astype(np.float64)
        if not np.array_equal(C, want):
            bad.append(("one_hot", K))
        # and with -1.5: C = -1.5 * W exactly (binary32 * 1.5 fits binary64)
        A2 = np.where(A == ONE, M1P5, np.uint16(0))
        if not np.array_equal(gemm(A2, W, K), -1.5 * want):
            bad.append(("one_hot_scaled", K))
    return bad


def pin_reduces_to_bf16_oracle(gemm):
    bad = []
    rng = np.random.default_rng(11)
    for (M, N, K) in ((1, 7, 33), (16, 40, 2880), (5, 3, 7168)):
        A = _rand_a(rng, (M, K))
        B = _rand_a(rng, (N, K))
        W = oracle.bf16_decode(B).astype(np.float32)  # exact: bf16 values are binary32
        if not np.array_equal(gemm(A, W, K), oracle.gemm_f64(A, B, K)):
            bad.append(("bf16_weights", M, N, K))
    return bad


def pin_constant(gemm):
    bad = []
    cases = [(ONE, np.float32(1.0 + 2.0 ** -20), 1.0), (M1P5, np.float32(0.75 + 2.0 ** -22), -1.5)]
    for K in (1, 1536, 2880, 7168, 14336):
        for (abits, w, a) in cases:
            A = np.full((2, K), abits, np.uint16)
            W = np.full((3, K), w, np.float32)
            want = float(Fraction(K) * Fraction(a) * Fraction(float(w)))
            C = gemm(A, W, K)
            if not np.all(C == want):
                bad.append(("constant", K, a))
    return bad


def pin_bruteforce(gemm, n_cases=30):
    bad = []
    rng = np.random.default_rng(12)
    u = 2.0 ** -53
    for i in range(n_cases):
        M, N, K = int(rng.integers(1, 5)), int(rng.integers(1, 6)), int(rng.integers(1, 70))
        A = _rand_a(rng, (M, K))
        W = _rand_w(rng, (N, K), 0.3)
        C = gemm(A, W, K)
        Ad = oracle.bf16_decode(A)
        for m in range(M):
            for n in range(N):
                exact = sum(Fraction(float(Ad[m, k])) * Fraction(float(W[n, k])) for k in range(K))
                absum = sum(abs(float(Ad[m, k]) * float(W[n, k])) for k in range(K))
                g = (K - 1) * u / (1 - (K - 1) * u)
                if abs(Fraction(float(C[m, n])) - exact) > Fraction(g * absum) + Fraction(0):
                    bad.append(("bruteforce", i, m, n))
    return bad


def pin_numpy(gemm):
    bad = []
    rng = np.random.default_rng(13)
    for (M, N, K) in ((16, 64, 7168), (3, 128, 2880), (1, 256, 7168)):
        A = _rand_a(rng, (M, K))
        W = _rand_w(rng, (N, K), 1 / np.sqrt(K))
        Ad = oracle.bf16_decode(A)
        ref = Ad @ W.astype(np.float64).T
        den = np.linalg.norm(Ad, axis=1)[:, None] * np.linalg.norm(W.astype(np.float64), axis=1)[None, :]
        if np.max(np.abs(gemm(A, W, K) - ref) / den) > 1e-12:
            bad.append(("numpy", M, N, K))
    return bad


def pin_padding(gemm):
    rng = np.random.default_rng(14)
    K, lda, ldw = 37, 48, 44
    A = np.full((3, lda), np.uint16(0x7FC1), np.uint16)
    A[:, :K] = _rand_a(rng, (3, K))
    W = np.full((5, ldw), np.float32("nan"), np.float32)
    W[:, :K] = _rand_w(rng, (5, K))
    C = gemm(A, W, K)
    ok = np.isfinite(C).all() and np.array_equal(C, gemm(np.ascontiguousarray(A[:, :K]),
                                                          np.ascontiguousarray(W[:, :K]), K))
    return [] if ok else [("padding",)]


def pin_degenerate(gemm):
    bad = []
    A = np.zeros((2, 4), np.uint16)
    W = np.ones((3, 4), np.float32)
    if not np.array_equal(gemm(A, W, 0), np.zeros((2, 3))):
        bad.append(("K0",))
    if gemm(np.zeros((0, 4), np.uint16), W, 4).shape != (0, 3):
        bad.append(("M0",))
    if gemm(A, np.zeros((0, 4), np.float32), 4).shape != (2, 0):
        bad.append(("N0",))
    return bad


PINS = [pin_one_hot, pin_reduces_to_bf16_oracle, pin_constant, pin_bruteforce, pin_numpy,
        pin_padding, pin_degenerate]


def _c(A, W, K):
    return oracle.gemm_f32w(A, W, K)


def _py(A, W, K):
    M, N = np.asarray(A).shape[0], np.asarray(W).shape[0]
    return np.array(oracle.gemm_f32w_py(A, W, K), dtype=np.float64).reshape(M, N)


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_c_oracle_f32w_pins(pin):
    assert pin(_c) == []


@pytest.mark.parametrize("pin", [pin_bruteforce, pin_padding, pin_degenerate],
                         ids=lambda p: p.__name__)
def test_python_oracle_f32w_pins(pin):
    assert pin(_py) == []


def test_points_match_full_f32w():
    rng = np.random.default_rng(15)
    A = _rand_a(rng, (5, 333))
    W = _rand_w(rng, (21, 333))
    C = oracle.gemm_f32w(A, W, 333)
    ms, ns = rng.integers(0, 5, 30), rng.integers(0, 21, 30)
    assert np.array_equal(oracle.gemm_f32w_points(A, W, 333, ms, ns), C[ms, ns])


# ---- planted mistakes --------------------------------------------------------

def weights_rounded_to_bf16(A, W, K):
    Wb = np.asarray(W, np.float32).view(np.uint32)
    Wb = ((Wb + np.uint32(0x7FFF) + ((Wb >> 16) & 1)) >> 16).astype(np.uint16)
    return oracle.gemm_f64(A, Wb, K)


def weights_truncated_to_bf16(A, W, K):
    return oracle.gemm_f64(A, (np.asarray(W, np.float32).view(np.uint32) >> 16).astype(np.uint16), K)


def fp32_accumulation(A, W, K):
    Ad = oracle.bf16_decode(np.asarray(A)[:, :K]).astype(np.float32)
    Wf = np.asarray(W, np.float32)[:, :K]
    C = np.zeros((Ad.shape[0], Wf.shape[0]), np.float32)
    for k in range(K):
        C = C + np.outer(Ad[:, k], Wf[:, k]).astype(np.float32)
    return C.astype(np.float64)


def drop_last_term(A, W, K):
    return oracle.gemm_f32w(A, W, max(K - 1, 0))


def w_index_off_by_one(A, W, K):
    return oracle.gemm_f32w(A, np.ascontiguousarray(np.roll(W, -1, axis=1)), K)


def wrong_sign(A, W, K):
    return -oracle.gemm_f32w(A, W, K)


def products_in_fp32(A, W, K):
    # each product rounded to binary32 before a binary64 sum
    Ad = oracle.bf16_decode(np.asarray(A)[:, :K]).astype(np.float32)
    Wf = np.asarray(W, np.float32)[:, :K]
    P = (Ad[:, None, :] * Wf[None, :, :]).astype(np.float32).astype(np.float64)
    return P.sum(axis=2)


MUTANTS = [weights_rounded_to_bf16, weights_truncated_to_bf16, fp32_accumulation, drop_last_term,
           w_index_off_by_one, wrong_sign, products_in_fp32]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda m: m.__name__)
def test_f32w_mutant_is_caught(mutant):
    caught = []
    for pin in (pin_one_hot, pin_constant, pin_bruteforce, pin_reduces_to_bf16_oracle):
        try:
            if pin(mutant):
                caught.append(pin.__name__)
        except Exception:
            caught.append(pin.__name__ + " (raised)")
    assert caught, mutant.__name__

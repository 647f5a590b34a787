"""Planted mistakes in the oracle must be caught by the pins (CPU only).

Each mutant is the real oracle with one plausible slip planted around it; the
pins in ``oracle_pins`` must reject every one of them, while accepting the
real oracle (``test_oracle_pins``)."""
import numpy as np
import pytest

import oracle
from tests import oracle_pins as pins


def _g(A, B, K):
    return oracle.gemm_f64(A, B, K)


def drop_last_term(A, B, K):
    return _g(A, B, max(K - 1, 0))


def drop_first_term(A, B, K):
    if K == 0:
        return _g(A, B, 0)
    return _g(np.ascontiguousarray(A[:, 1:]), np.ascontiguousarray(B[:, 1:]), K - 1)


def b_index_off_by_one(A, B, K):
    return _g(A, np.ascontiguousarray(np.roll(B, -1, axis=1)), K)


def b_transposed(A, B, K):
    # read B[n, k] from storage position k * N + n (column-major slip)
    N, ldb = B.shape
    flat = np.ascontiguousarray(B).reshape(-1)
    if N == 0 or K == 0:
        return _g(A, B, K)
    idx = (np.arange(K)[None, :] * N + np.arange(N)[:, None]) % flat.size
    return _g(A, np.ascontiguousarray(flat[idx]), K)


def a_uses_b_stride(A, B, K):
    M, lda = A.shape
    ldb = B.shape[1]
    if lda == ldb or M == 0:
        return _g(A, B, K)
    flat = np.concatenate([np.ascontiguousarray(A).reshape(-1), np.zeros(M * ldb, np.uint16)])
    A2 = np.stack([flat[m * ldb: m * ldb + lda] for m in range(M)])
    return _g(A2, B, K)


def wrong_sign(A, B, K):
    return -_g(A, B, K)


def drop_sign_bit(A, B, K):
    return _g(A & np.uint16(0x7FFF), B, K)


def fp16_decode(A, B, K):
    Ad = np.asarray(A, np.uint16)[:, :K].view(np.float16).astype(np.float64)
    Bd = np.asarray(B, np.uint16)[:, :K].view(np.float16).astype(np.float64)
    return Ad @ Bd.T


def fp32_accumulate(A, B, K):
    Ad = oracle.bf16_decode(np.asarray(A)[:, :K]).astype(np.float32)
    Bd = oracle.bf16_decode(np.asarray(B)[:, :K]).astype(np.float32)
    M, N = Ad.shape[0], Bd.shape[0]
    C = np.zeros((M, N), dtype=np.float32)
    for k in range(K):
        C += np.outer(Ad[:, k], Bd[:, k])
    return C.astype(np.float64)


def output_transposed(A, B, K):
    return _g(B, A, K)


def ignores_last_row_of_b(A, B, K):
    C = _g(A, B, K)
    if C.shape[1]:
        C[:, -1] = 0.0
    return C


MUTANTS = [drop_last_term, drop_first_term, b_index_off_by_one, b_transposed,
           a_uses_b_stride, wrong_sign, drop_sign_bit, fp16_decode, fp32_accumulate,
           output_transposed, ignores_last_row_of_b]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda f: f.__name__)
def test_mutant_is_caught(mutant):
    fails = pins.run_all(mutant)
    assert fails, f"no pin caught the planted mistake {mutant.__name__}"

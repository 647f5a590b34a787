"""The oracle against what the mathematics fixes (CPU only)."""
import os

import numpy as np
import pytest

import oracle
from oracle import acceptance
from tests import oracle_pins as pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _c_gemm(A, B, K):
    return oracle.gemm_f64(A, B, K)


def _py_gemm(A, B, K):
    C = oracle.gemm_py(A, B, K)
    return np.array(C, dtype=np.float64).reshape(np.asarray(A).shape[0], np.asarray(B).shape[0])


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_c_oracle_pins(pin):
    assert pin(_c_gemm) == []


@pytest.mark.parametrize("pin", [pins.pin_one_hot, pins.pin_constant, pins.pin_padding,
                                 pins.pin_degenerate, pins.pin_invariants],
                         ids=lambda p: p.__name__)
def test_python_oracle_pins(pin):
    assert pin(_py_gemm) == []


def test_python_and_c_loops_agree_bitwise():
    # same k order, exact products, binary64 sums: identical bits expected
    rng = np.random.default_rng(1)
    for (M, N, K) in ((1, 1, 1), (3, 7, 40), (16, 5, 129), (2, 3, 0)):
        A = pins._rand_bits(rng, (M, max(K, 1)))
        B = pins._rand_bits(rng, (N, max(K, 1)))
        assert np.array_equal(_py_gemm(A, B, K), _c_gemm(A, B, K))


def test_points_match_full():
    rng = np.random.default_rng(2)
    M, N, K = 6, 50, 777
    A = pins._rand_bits(rng, (M, K))
    B = pins._rand_bits(rng, (N, K))
    C = oracle.gemm_f64(A, B, K)
    ms = rng.integers(0, M, 40)
    ns = rng.integers(0, N, 40)
    assert np.array_equal(oracle.gemm_points(A, B, K, ms, ns), C[ms, ns])


def test_threads_do_not_change_bits():
    rng = np.random.default_rng(3)
    A = pins._rand_bits(rng, (4, 1000))
    B = pins._rand_bits(rng, (37, 1000))
    assert np.array_equal(oracle.gemm_f64(A, B, 1000, threads=1), oracle.gemm_f64(A, B, 1000, threads=5))


def _golden_rne():
    rows = []
    with open(os.path.join(GOLDEN, "bf16_rne.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            rows.append((float.fromhex(parts[0]), int(parts[1], 16), " ".join(parts[2:])))
    return rows


@pytest.mark.parametrize("value,bits,why", _golden_rne())
def test_round_bf16_golden(value, bits, why):
    assert oracle.round_bf16(value) == bits, why


def test_round_bf16_nan_inf():
    assert oracle.round_bf16(float("inf")) == 0x7F80
    assert oracle.round_bf16(float("-inf")) == 0xFF80
    r = oracle.round_bf16(float("nan"))
    assert (r & 0x7F80) == 0x7F80 and (r & 0x7F) != 0


def test_round_bf16_exhaustive_representables():
    # every finite bf16 value rounds to itself
    bits = np.arange(0x10000, dtype=np.uint32).astype(np.uint16)
    vals = oracle.bf16_decode(bits)
    finite = np.isfinite(vals)
    for b, v in zip(bits[finite][::97], vals[finite][::97]):
        got = oracle.round_bf16(float(v))
        if v == 0.0:
            assert (got & 0x7FFF) == 0
        else:
            assert got == int(b)


def test_decode_matches_format_arithmetic():
    bits = np.arange(0x10000, dtype=np.uint32).astype(np.uint16)
    v = oracle.bf16_decode(bits)
    w = pins._dec(bits)
    fin = np.isfinite(v)
    assert np.array_equal(v[fin], w[fin])
    assert np.all(np.isinf(v[(bits & 0x7FFF) == 0x7F80]))


def test_acceptance_measures():
    C_ref = np.array([[1.0, 0.0], [2.0, 0.0]])
    an = np.array([1.0, 2.0])
    bn = np.array([1.0, 0.0])
    C = C_ref.copy()
    assert acceptance.normalized_error(C, C_ref, an, bn) == 0.0
    C[1, 0] += 0.003          # denominator 2*1 -> 0.0015
    assert abs(acceptance.normalized_error(C, C_ref, an, bn) - 0.0015) < 1e-15
    C2 = C_ref.copy()
    C2[0, 1] = 1e-30          # a zero denominator needs an exact zero
    assert acceptance.normalized_error(C2, C_ref, an, bn) == float("inf")
    C3 = C_ref.copy()
    C3[0, 0] = np.nan
    assert acceptance.normalized_error(C3, C_ref, an, bn) == float("inf")
    cos = acceptance.row_cosines(np.array([[1.0, 0.0], [0.0, 0.0]]), np.array([[2.0, 0.0], [0.0, 0.0]]))
    assert cos[0] == 1.0 and cos[1] == 1.0
    assert acceptance.row_cosines(np.array([[0.0, 0.0]]), np.array([[1.0, 0.0]]))[0] == 0.0
    assert acceptance.assess(C, C_ref, an, bn, "f32")["ok"]
    C[1, 0] += 0.006          # now 0.0045 > 2e-3 but < 1e-2
    assert not acceptance.assess(C, C_ref, an, bn, "f32")["ok"]
    assert acceptance.assess(C, C_ref, an, bn, "bf16")["ok"]

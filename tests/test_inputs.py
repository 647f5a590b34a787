"""Seeded input generator (CPU only)."""
import numpy as np

import oracle
from latency_decode_gemm_amd import inputs


def test_deterministic_and_seeded():
    a1 = inputs.make_a(4, 300, 128)
    a2 = inputs.make_a(4, 300, 128)
    assert np.array_equal(a1, a2)
    b0 = inputs.make_b(300, 128, r=0)
    b1 = inputs.make_b(300, 128, r=1)
    assert not np.array_equal(b0, b1)
    assert inputs.seed_a(1, 7168, 256) == 1_000_003 * 7168 + 10_007 * 256 + 1
    assert inputs.seed_b(7168, 256, 3) == 7_919 * 7168 + 104_729 * 256 + 3


def test_distribution():
    K = 4096
    b = oracle.bf16_decode(inputs.make_b(K, 64))
    a = oracle.bf16_decode(inputs.make_a(8, K, 64))
    assert abs(a.std() - 1.0) < 0.02 and abs(a.mean()) < 0.02
    assert abs(b.std() * np.sqrt(K) - 1.0) < 0.02


def test_padding_is_nan_pattern():
    a = inputs.make_a(3, 45, 10, lda=56)
    assert np.all(a[:, 45:] == inputs.PAD_BITS)
    assert np.all(np.isfinite(oracle.bf16_decode(a[:, :45])))
    assert np.isnan(oracle.bf16_decode(a[:, 50])).all()


def test_bf16_quantisation_is_nearest_even():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(2000) * 10.0 ** rng.integers(-30, 30, 2000)).astype(np.float32)
    x = np.concatenate([x, np.float32([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 0.0, -0.0])])
    got = inputs.f32_to_bf16_bits(x)
    want = np.array([oracle.round_bf16(float(v)) for v in x], dtype=np.uint16)
    assert np.array_equal(got, want)


def test_workload_points():
    pts = inputs.all_points()
    assert len(pts) == 29
    assert sum(1 for p in pts if p["out"] == "bf16") == 14
    assert all(p["M"] <= 16 for p in pts)


def test_f32_weights_are_the_unrounded_draws():
    from latency_decode_gemm_amd import inputs
    W = inputs.make_w_f32(100, 7, ldw=104)
    B = inputs.make_b(100, 7, ldb=104)
    assert W.dtype == np.float32 and W.shape == (7, 104)
    assert np.array_equal(inputs.f32_to_bf16_bits(W[:, :100]), B[:, :100])
    assert np.isnan(W[:, 100:]).all()
    # the draws use every bit of the binary32 significand
    assert (W[:, :100].view(np.uint32) & 0xFFFF).any()

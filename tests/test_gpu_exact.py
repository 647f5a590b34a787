"""Bit-exact cases on the GPU (inputs whose fp32 sums are exact in any order).

One-hot rows of A pick single columns of B, B = I returns A, constants give
K*a*b, and small dyadic inputs give exact sums whose bf16 rounding is
compared bit for bit with the oracle's nearest-even rounding.  These pin the
lane layouts of every kernel family (including the MFMA operand and result
layouts) and the bf16 epilogue exactly."""
import numpy as np
import pytest

import oracle
import latency_decode_gemm_amd as skg
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

MK = skg.SkgConfig.make
V, F, GA = skg.SKG_INNER_VALU, skg.SKG_INNER_MFMA, skg.SKG_INNER_MFMA_GA
VG = skg.SKG_INNER_VALU_GA
RF, RG = skg.SKG_INNER_MFMA_RING, skg.SKG_INNER_MFMA_RING_GA
SY, SH = skg.SKG_INNER_MFMA_RING_SYNC, skg.SKG_INNER_MFMA_RING_SHARED

FAMILIES = [
    None,  # the dispatch table's choice
    MK(inner=V, split_k=1, row_tiles=1, waves_n=1, waves_k=1, depth=4),
    MK(inner=V, split_k=1, row_tiles=2, waves_n=2, waves_k=4, depth=4),
    MK(inner=V, split_k=3, row_tiles=4, waves_n=1, waves_k=2, depth=2),
    MK(inner=F, split_k=1, row_tiles=1, waves_n=1, waves_k=1, depth=4),
    MK(inner=F, split_k=1, row_tiles=2, waves_n=2, waves_k=4, depth=2),
    MK(inner=F, split_k=4, row_tiles=4, waves_n=1, waves_k=2, depth=1),
    MK(inner=GA, split_k=1, row_tiles=1, waves_n=1, waves_k=4, depth=3, rb_per_wg=2),
    MK(inner=GA, split_k=2, row_tiles=2, waves_n=2, waves_k=1, depth=1),
    MK(backend=skg.SKG_BACKEND_SPLITK_2PASS, inner=GA, split_k=3, row_tiles=1, waves_n=1,
       waves_k=2, depth=2),
    MK(backend=skg.SKG_BACKEND_SPLITK_2PASS, inner=V, split_k=2, row_tiles=2, waves_n=1,
       waves_k=2, depth=4),
    MK(inner=VG, split_k=1, row_tiles=1, waves_n=1, waves_k=1, depth=4),
    MK(inner=VG, split_k=1, row_tiles=2, waves_n=2, waves_k=4, depth=4),
    MK(backend=skg.SKG_BACKEND_SPLITK_2PASS, inner=VG, split_k=3, row_tiles=4, waves_n=1,
       waves_k=2, depth=2),
    MK(inner=RF, split_k=1, row_tiles=1, waves_n=2, waves_k=2, depth=4),
    MK(backend=skg.SKG_BACKEND_EVEN, inner=V, split_k=1, row_tiles=2, waves_n=2, waves_k=2,
       depth=4),
    MK(backend=skg.SKG_BACKEND_EVEN, inner=GA, split_k=1, row_tiles=1, waves_n=2, waves_k=1,
       depth=3),
    MK(inner=RF, split_k=2, row_tiles=2, waves_n=1, waves_k=1, depth=2),
    MK(inner=RG, split_k=1, row_tiles=2, waves_n=1, waves_k=2, depth=3),
    MK(backend=skg.SKG_BACKEND_SPLITK_2PASS, inner=RG, split_k=3, row_tiles=1, waves_n=2,
       waves_k=1, depth=6),
    MK(inner=SY, split_k=1, row_tiles=1, waves_n=3, waves_k=1, depth=3, rb_per_wg=2),
    MK(inner=SH, split_k=1, row_tiles=1, waves_n=3, waves_k=1, depth=4, rb_per_wg=2),
    MK(backend=skg.SKG_BACKEND_EVEN, inner=SH, split_k=1, row_tiles=2, waves_n=1, waves_k=2,
       depth=3),
    MK(inner=SH, split_k=3, row_tiles=1, waves_n=2, waves_k=2, depth=3),
]


def _first_fit(cfg, M, shapes):
    """The first (K, N) in shapes that the configuration runs (all fit the
    dispatch table's choice)."""
    for K, N in shapes:
        if cfg is None or skg.skinny_gemm_check_config(M, K, N, cfg):
            return K, N
    raise AssertionError(f"no test shape fits {cfg}")


def _m_for(cfg, m):
    """Tokens for a test shape: the activation-ring VALU kernel takes M <= 8."""
    return min(m, 8) if cfg is not None and cfg.inner == VG else m


def _fid(c):
    if c is None:
        return "dispatch"
    return ("p2_" if c.backend == 2 else "ev_" if c.backend == 3 else "") + \
        {V: "valu", F: "mfma", GA: "mfmaga", VG: "valuga", RF: "ring", RG: "ringga",
         SY: "ringsync", SH: "ringshared"}[c.inner] + \
        f"_S{c.split_k}_r{c.row_tiles}_n{c.waves_n}_k{c.waves_k}_b{c.rb_per_wg}_d{c.depth}"


def _gemm(A, B, cfg, out_dtype):
    if cfg is None:
        return skg.skinny_gemm_bf16(A, B, out_dtype=out_dtype)
    return skg.skinny_gemm_bf16_with_config(A, B, cfg, out_dtype=out_dtype)


def _dyadic(rng, shape, lo, hi, scale):
    v = rng.integers(lo, hi + 1, size=shape).astype(np.float64) * scale
    bits = np.array([oracle.round_bf16(x) for x in v.ravel()], dtype=np.uint16).reshape(shape)
    assert np.array_equal(oracle.bf16_decode(bits), v)  # exactly representable
    return bits


@pytest.mark.parametrize("cfg", FAMILIES, ids=_fid)
def test_one_hot(cfg):
    """Every family runs every one-hot position of at least one ragged K
    (main steps, the last full chunk, the chunk that straddles K), in groups
    of as many tokens as the family takes; each of K = 2880, 1531 and 1003
    where the family fits it."""
    torch = gu.torch_cuda()
    rng = np.random.default_rng(7)
    N = 48
    ran = {}
    for K, ks in ((2880, [0, 7, 8, 127, 128, 2047, 2048, 2559, 2560, 2687, 2688, 2815,
                          2816, 2871, 2872, 2879]),
                  (1531, [0, 7, 8, 127, 128, 1023, 1024, 1407, 1408, 1519, 1520, 1523,
                          1524, 1527, 1528, 1530]),
                  (1003, [0, 1, 8, 500, 999, 1000, 1001, 1002])):
        ld = gu.round8(K)
        B_bits = np.full((N, ld), 0x7FC1, dtype=np.uint16)
        B_bits[:, :K] = _dyadic(rng, (N, K), -255, 255, 2.0 ** -7)
        per = _m_for(cfg, len(ks))
        for g0 in range(0, len(ks), per):
            kg = ks[g0:g0 + per]
            M = len(kg)
            if cfg is not None and not skg.skinny_gemm_check_config(M, K, N, cfg):
                continue
            A_bits = np.zeros((M, ld), dtype=np.uint16)
            for m, k in enumerate(kg):
                A_bits[m, k] = 0x3F80
            A, B = gu.operands(A_bits, B_bits, K)
            C = _gemm(A, B, cfg, torch.float32)
            torch.cuda.synchronize()
            want = oracle.bf16_decode(B_bits[:, kg]).T
            got = gu.to_f64(C)
            assert np.array_equal(got, want), (K, kg, np.argwhere(got != want)[:8])
            ran[K] = ran.get(K, 0) + M
    # every position of some ragged K must have run (none may pass vacuously)
    assert ran.get(2880, 0) == 16 or ran.get(1531, 0) == 16, f"one-hot positions run: {ran}"


@pytest.mark.parametrize("cfg", FAMILIES, ids=_fid)
def test_identity(cfg):
    torch = gu.torch_cuda()
    rng = np.random.default_rng(8)
    M = _m_for(cfg, 16)
    # the smallest square that the configuration fits (a K split needs
    # enough K steps per slice)
    K = N = _first_fit(cfg, M, [(k, k) for k in (256, 1024, 2048)])[0]
    A_bits = _dyadic(rng, (M, K), -127, 127, 2.0 ** -3)
    B_bits = np.zeros((N, K), dtype=np.uint16)
    B_bits[np.arange(K), np.arange(K)] = 0x3F80
    A, B = gu.operands(A_bits, B_bits, K)
    for odt in (torch.float32, torch.bfloat16):
        C = _gemm(A, B, cfg, odt)
        torch.cuda.synchronize()
        assert np.array_equal(gu.to_f64(C), oracle.bf16_decode(A_bits))


@pytest.mark.parametrize("cfg", FAMILIES, ids=_fid)
def test_constant_closed_form(cfg):
    torch = gu.torch_cuda()
    ran = 0
    # 1 * 2^-6 summed K times, and -1.5 * 0.75 summed K times
    for K, ab, bb, want in ((7168, 0x3F80, 0x3C80, 112.0), (2880, 0x3F80, 0x3C80, 45.0),
                            (1536, 0x3F80, 0x3C80, 24.0), (7168, 0xBFC0, 0x3F40, -8064.0),
                            (512, 0x3F80, 0x3C80, 8.0), (256, 0xBFC0, 0x3F40, -288.0)):
        M, N = 5, 40
        if cfg is not None and not skg.skinny_gemm_check_config(M, K, N, cfg):
            continue
        ran += 1
        A_bits = np.full((M, K), ab, dtype=np.uint16)
        B_bits = np.full((N, K), bb, dtype=np.uint16)
        A, B = gu.operands(A_bits, B_bits, K)
        for odt in (torch.float32, torch.bfloat16):
            C = _gemm(A, B, cfg, odt)
            torch.cuda.synchronize()
            assert np.all(gu.to_f64(C) == want), (K, odt)
    assert ran >= 2, "fewer than two constant cases fit this configuration"


@pytest.mark.parametrize("cfg", FAMILIES, ids=_fid)
def test_bf16_rounding_is_nearest_even(cfg):
    """Exact dyadic sums: the bf16 output must be the nearest-even bf16 of the
    exact value (the oracle's rounding), bit for bit; ties included."""
    torch = gu.torch_cuda()
    rng = np.random.default_rng(9)
    # |A| <= 16, |B| <= 255 * 2^-8: every partial sum over K <= 4096 terms is
    # a multiple of 2^-8 below 2^16, exact in fp32 in any order
    M = _m_for(cfg, 16)
    K, N = _first_fit(cfg, M, [(48, 96), (384, 96), (1536, 96), (4096, 96)])
    A_bits = _dyadic(rng, (M, K), -16, 16, 1.0)
    B_bits = _dyadic(rng, (N, K), -255, 255, 2.0 ** -8)
    # hand-made ties in the first columns: 1 + 2^-8 -> 1.0, 1 + 3*2^-8 -> 1 + 2^-6
    A_bits[0, :] = 0
    A_bits[0, :2] = 0x3F80
    B_bits[0, :] = 0
    B_bits[0, :2] = [0x3F80, oracle.round_bf16(2.0 ** -8)]
    B_bits[1, :] = 0
    B_bits[1, :2] = [0x3F80, oracle.round_bf16(3 * 2.0 ** -8)]
    A, B = gu.operands(A_bits, B_bits, K)
    C = _gemm(A, B, cfg, torch.bfloat16)
    torch.cuda.synchronize()
    ref = oracle.gemm_f64(A_bits, B_bits, K)
    want = np.array([oracle.round_bf16(x) for x in ref.ravel()], dtype=np.uint16).reshape(M, N)
    got = gu.bits_of(C)
    assert got[0, 0] == 0x3F80 and got[0, 1] == 0x3F82
    assert np.array_equal(got, want), np.argwhere(got != want)[:8]
    # and the fp32 output is the exact sum
    C32 = _gemm(A, B, cfg, torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(gu.to_f64(C32), ref)

"""The router GEMM over fp32 weights (bf16 A, fp32 W) against the fp32-weight
oracle, element by element (GPU).

* the router shapes (K = 7168, N in {256, 384}, M in {1, 2, 3, 4, 8, 16}) at
  full size with the dispatched configuration, and every M = 1..16 on them
  (the untuned M take the entry of the next larger tuned M);
* every VALU variant and backend forced through the explicit-config entry on
  shapes with ragged K and N tails, NaN-padded leading dimensions;
* exact cases: one-hot activation rows select fp32 weights bit for bit (any
  rounding of W to bf16 would show), K < 8, K = 0;
* repeated calls and warm-up leave the bits unchanged.
"""
import numpy as np
import pytest

import oracle
import latency_decode_gemm_amd as skg
from latency_decode_gemm_amd import inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

MK = skg.SkgConfig.make
V, VG = skg.SKG_INNER_VALU, skg.SKG_INNER_VALU_GA
P2, EV = skg.SKG_BACKEND_SPLITK_2PASS, skg.SKG_BACKEND_EVEN


def _round4(x):
    return (x + 3) // 4 * 4


@pytest.mark.parametrize("p", inputs.WORKLOADS_F32W["router_f32w"],
                         ids=lambda p: f"M{p['M']}_K{p['K']}_N{p['N']}")
def test_router_f32w_point(p):
    torch = gu.torch_cuda()
    M, K, N = p["M"], p["K"], p["N"]
    A_bits = inputs.make_a(M, K, N)
    W = inputs.make_w_f32(K, N)
    A, Wd = gu.operands_f32w(A_bits, W, K)
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    skg.skinny_gemm_f32w(A, Wd, out=C)
    torch.cuda.synchronize()
    r = gu.assess_f32w(C, A_bits, W, K)
    assert r["ok"], r


@pytest.mark.parametrize("M", list(range(1, 17)))
@pytest.mark.parametrize("N", [256, 384])
def test_router_f32w_every_m(N, M):
    torch = gu.torch_cuda()
    K = 7168
    A_bits = inputs.make_a(M, K, N)
    W = inputs.make_w_f32(K, N)
    A, Wd = gu.operands_f32w(A_bits, W, K)
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    cfg = skg.skinny_gemm_f32w_dispatch(M, K, N)
    print(f"M={M} K={K} N={N} cfg={cfg.as_tuple()}", flush=True)
    skg.skinny_gemm_f32w(A, Wd, out=C)
    torch.cuda.synchronize()
    r = gu.assess_f32w(C, A_bits, W, K)
    assert r["ok"], (M, N, cfg.as_tuple(), r)


def _configs():
    out = []
    for (R, PF) in skg._capi.VALU_VARIANTS:
        out += [MK(inner=V, split_k=1, row_tiles=R, waves_n=1, waves_k=1, depth=PF),
                MK(inner=V, split_k=1, row_tiles=R, waves_n=2, waves_k=3, depth=PF, rb_per_wg=3),
                MK(inner=V, split_k=3, row_tiles=R, waves_n=1, waves_k=2, depth=PF, rb_per_wg=2),
                MK(backend=P2, inner=V, split_k=2, row_tiles=R, waves_n=2, waves_k=1, depth=PF),
                MK(inner=VG, split_k=1, row_tiles=R, waves_n=1, waves_k=1, depth=PF),
                MK(inner=VG, split_k=3, row_tiles=R, waves_n=1, waves_k=2, depth=PF, rb_per_wg=2),
                MK(backend=EV, inner=V, split_k=1, row_tiles=R, waves_n=2, waves_k=2, depth=PF),
                MK(backend=EV, inner=VG, split_k=4, row_tiles=R, waves_n=1, waves_k=1, depth=PF)]
    return out


SHAPES = [(1, 2880, 200), (3, 1003, 77), (8, 4104, 130), (16, 2880, 128), (16, 777, 33),
          (5, 7168, 100), (11, 520, 50), (2, 9, 5), (13, 33, 300)]


def _cfg_id(c):
    return ("p2_" if c.backend == P2 else "ev_" if c.backend == EV else "") + \
        {V: "valu", VG: "valuga"}[c.inner] + \
        f"_S{c.split_k}_r{c.row_tiles}_n{c.waves_n}_k{c.waves_k}_d{c.depth}_b{c.rb_per_wg}"


@pytest.mark.parametrize("cfg", _configs(), ids=_cfg_id)
def test_f32w_forced_config(cfg):
    torch = gu.torch_cuda()
    ran = 0
    for (M, K, N) in SHAPES:
        lda, ldw = gu.round8(K) + 8, _round4(K) + 4   # NaN padding on both operands
        A_bits = inputs.make_a(M, K, N, lda=lda)
        W = inputs.make_w_f32(K, N, ldw=ldw)
        A, Wd = gu.operands_f32w(A_bits, W, K)
        for out_dtype in (torch.float32, torch.bfloat16):
            if not skg.skinny_gemm_f32w_check_config(M, K, N, cfg):
                with pytest.raises(skg.SkinnyGemmError):
                    skg.skinny_gemm_f32w_with_config(A, Wd, cfg, out_dtype=out_dtype)
                continue
            C = skg.skinny_gemm_f32w_with_config(A, Wd, cfg, out_dtype=out_dtype)
            torch.cuda.synchronize()
            r = gu.assess_f32w(C, A_bits, W, K)
            assert r["ok"], (M, K, N, out_dtype, r)
            ran += 1
    assert ran > 0


@pytest.mark.parametrize("shape", [(16, 2880, 200), (3, 1003, 77), (1, 7168, 256), (9, 8, 40)],
                         ids=lambda s: "M%d_K%d_N%d" % s)
def test_f32w_one_hot_selects_weights_exactly(shape):
    """A[m, :] = e_{k_m}: C[m, n] = W[n, k_m] exactly in fp32, and its nearest
    even bf16 for bf16 output (positions include the ragged end of K)."""
    torch = gu.torch_cuda()
    M, K, N = shape
    ks = [min(K - 1, k) for k in (0, K - 1, K // 2, 2047, 2559, 7, 8, 129, 1000, 2879, 3, 5,
                                  K - 2, K - 3, 64, 127)][:M]
    lda = gu.round8(K)
    A_bits = np.zeros((M, lda), np.uint16)
    for m, k in enumerate(ks):
        A_bits[m, k] = 0x3F80
    W = inputs.make_w_f32(K, N, ldw=_round4(K))
    A, Wd = gu.operands_f32w(A_bits, W, K)
    C = skg.skinny_gemm_f32w(A, Wd)
    Cb = skg.skinny_gemm_f32w(A, Wd, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    want = np.ascontiguousarray(W[:, ks].T)
    assert np.array_equal(gu.bits_of(C), want.view(np.uint32))
    want_b = np.array([[oracle.round_bf16(float(v)) for v in row] for row in want], np.uint16)
    assert np.array_equal(gu.bits_of(Cb), want_b)


@pytest.mark.parametrize("K", [0, 1, 2, 3, 5, 7, 8, 9, 15, 17])
def test_f32w_short_k(K):
    torch = gu.torch_cuda()
    M, N = 4, 37
    ld = max(8, gu.round8(K))
    A_bits = inputs.make_a(M, K, N, lda=ld)
    W = inputs.make_w_f32(K, N, ldw=ld)
    A, Wd = gu.operands_f32w(A_bits, W, K)
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    skg.skinny_gemm_f32w(A, Wd, out=C)
    torch.cuda.synchronize()
    if K == 0:
        assert np.all(gu.to_f64(C) == 0.0)
    else:
        r = gu.assess_f32w(C, A_bits, W, K)
        assert r["ok"], r


def test_f32w_repeated_calls_and_warmup_identical():
    torch = gu.torch_cuda()
    shapes = [(7168, 256), (7168, 384)]
    ms = [1, 2, 3, 4, 8, 16]
    for (K, N) in shapes:
        for M in (3, 16):
            A_bits = inputs.make_a(M, K, N)
            W = inputs.make_w_f32(K, N)
            A, Wd = gu.operands_f32w(A_bits, W, K)
            ref = gu.bits_of(skg.skinny_gemm_f32w(A, Wd))
            outs = [skg.skinny_gemm_f32w(A, Wd) for _ in range(20)]
            torch.cuda.synchronize()
            for o in outs:
                assert np.array_equal(gu.bits_of(o), ref)
    n = skg.skinny_gemm_f32w_warmup(shapes, ms)
    assert n == len(skg.skinny_gemm_f32w_warmup_keys(shapes, ms))
    A_bits = inputs.make_a(16, 7168, 384)
    W = inputs.make_w_f32(7168, 384)
    A, Wd = gu.operands_f32w(A_bits, W, 7168)
    before = gu.bits_of(skg.skinny_gemm_f32w(A, Wd))
    assert skg.skinny_gemm_f32w_warmup(shapes, ms) == n
    after = gu.bits_of(skg.skinny_gemm_f32w(A, Wd))
    torch.cuda.synchronize()
    assert np.array_equal(before, after)


def test_f32w_dtype_guards():
    torch = gu.torch_cuda()
    A = torch.zeros((2, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(TypeError):
        skg.skinny_gemm_f32w(A, torch.zeros((3, 64), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(TypeError):
        skg.skinny_gemm_bf16(A, torch.zeros((3, 64), dtype=torch.float32, device="cuda"))

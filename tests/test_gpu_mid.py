"""The middle tier, 16 < M <= 64 (the matrix-core kernels with 2 to 4 token
tiles of 16), against the oracle element by element (GPU).

* the middle-tier workload (qkv_a-style into the ldc = 4096 bf16 buffer, the
  wide and the deep projection, M in {24, 32, 48, 64}) at full size with the
  dispatched configuration, on every row and sampled columns;
* every matrix-core kind and backend forced through the explicit-config entry
  on shapes with ragged M, K and N tails and NaN-padded leading dimensions;
* the LDS-ring kernels against the register-ring ones, bit for bit;
* repeated calls bit-identical.
"""
import numpy as np
import pytest

import latency_decode_gemm_amd as skg
from latency_decode_gemm_amd import inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

MK = skg.SkgConfig.make
F, GA = skg.SKG_INNER_MFMA, skg.SKG_INNER_MFMA_GA
RF, RG = skg.SKG_INNER_MFMA_RING, skg.SKG_INNER_MFMA_RING_GA
P2, EV = skg.SKG_BACKEND_SPLITK_2PASS, skg.SKG_BACKEND_EVEN

SHAPES = [(17, 2880, 200), (24, 1003, 77), (33, 4104, 130), (48, 777, 33), (64, 520, 50),
          (63, 33, 300), (40, 7168, 100), (64, 2880, 128), (49, 136, 1000)]


def _all_configs():
    out = []
    for (G, PF) in skg._capi.MFMA_VARIANTS:
        out += [MK(inner=F, split_k=1, row_tiles=G, waves_n=1, waves_k=1, depth=PF),
                MK(inner=F, split_k=4, row_tiles=G, waves_n=1, waves_k=2, depth=PF, rb_per_wg=2),
                MK(inner=GA, split_k=1, row_tiles=G, waves_n=2, waves_k=2, depth=PF, rb_per_wg=3),
                MK(inner=GA, split_k=3, row_tiles=G, waves_n=1, waves_k=2, depth=PF),
                MK(backend=P2, inner=GA, split_k=4, row_tiles=G, waves_n=1, waves_k=1, depth=PF),
                MK(inner=RF, split_k=2, row_tiles=G, waves_n=1, waves_k=2, depth=PF),
                MK(inner=RG, split_k=1, row_tiles=G, waves_n=2, waves_k=1, depth=PF),
                MK(inner=RG, split_k=3, row_tiles=G, waves_n=1, waves_k=2, depth=PF, rb_per_wg=2),
                MK(backend=EV, inner=RG, split_k=1, row_tiles=G, waves_n=1, waves_k=2, depth=PF),
                MK(backend=EV, inner=GA, split_k=2, row_tiles=G, waves_n=1, waves_k=1, depth=PF)]
    return out


def _runs(cfg):
    return sum(skg.skinny_gemm_check_config(M, K, N, cfg) for (M, K, N) in SHAPES)


# configurations that can run at least one shape (the combinations that would
# spill are not built, so some never can)
CONFIGS = [c for c in _all_configs() if _runs(c) > 0]


def _cfg_id(c):
    return ("p2_" if c.backend == P2 else "ev_" if c.backend == EV else "") + \
        {F: "mfma", GA: "mfmaga", RF: "ring", RG: "ringga"}[c.inner] + \
        f"_S{c.split_k}_r{c.row_tiles}_n{c.waves_n}_k{c.waves_k}_d{c.depth}_b{c.rb_per_wg}"


def test_most_configurations_run():
    assert len(CONFIGS) >= 0.6 * len(_all_configs())


@pytest.mark.parametrize("cfg", CONFIGS, ids=_cfg_id)
def test_mid_forced_config(cfg):
    torch = gu.torch_cuda()
    for (M, K, N) in SHAPES:
        if not skg.skinny_gemm_check_config(M, K, N, cfg):
            continue
        ld = gu.round8(K) + 8
        A_bits = inputs.make_a(M, K, N, lda=ld)
        B_bits = inputs.make_b(K, N, ldb=ld)
        A, B = gu.operands(A_bits, B_bits, K)
        for out_dtype in (torch.float32, torch.bfloat16):
            C = torch.full((M, N), float("nan"), dtype=out_dtype, device="cuda")
            print(f"case M={M} K={K} N={N} out={out_dtype}", flush=True)
            skg.skinny_gemm_bf16_with_config(A, B, cfg, out=C)
            torch.cuda.synchronize()
            r = gu.assess(C, A_bits, B_bits, K)
            assert r["ok"], (M, K, N, out_dtype, r)


@pytest.mark.parametrize("p", inputs.WORKLOADS_MID["mid_m"] + inputs.WORKLOADS_MID["mid_router"],
                         ids=lambda p: f"M{p['M']}_K{p['K']}_N{p['N']}")
def test_mid_workload_point(p):
    torch = gu.torch_cuda()
    M, K, N = p["M"], p["K"], p["N"]
    ldc = p["ldc"] or N
    A_bits = inputs.make_a(M, K, N)
    B_bits = gu.cached_b(K, N)
    A, B = gu.operands(A_bits, B_bits, K)
    dt = torch.bfloat16 if p["out"] == "bf16" else torch.float32
    buf = torch.full((M, ldc), float("nan"), dtype=dt, device="cuda")
    skg.skinny_gemm_bf16(A, B, out=buf[:, :N])
    torch.cuda.synchronize()
    r = gu.assess_sampled(buf[:, :N], A_bits, B_bits, K)
    assert r["ok"], r
    if ldc > N:
        assert np.isnan(gu.to_f64(buf[:, N:])).all()


@pytest.mark.parametrize("variant", list(skg._capi.MFMA_VARIANTS), ids=lambda v: f"G{v[0]}_d{v[1]}")
def test_mid_lds_ring_equals_register_ring(variant):
    """Same MFMAs on the same operands in the same order: identical bits."""
    torch = gu.torch_cuda()
    G, PF = variant
    for (M, K, N) in [(40, 1000, 333), (64, 2880, 200), (17, 136, 1000)]:
        ld = gu.round8(K)
        A_bits = inputs.make_a(M, K, N, lda=ld)
        B_bits = inputs.make_b(K, N, ldb=ld)
        A, B = gu.operands(A_bits, B_bits, K)
        for (reg, ring) in ((F, RF), (GA, RG)):
            for (S, wn, wk) in ((1, 1, 1), (2, 1, 2)):
                kw = dict(split_k=S, row_tiles=G, waves_n=wn, waves_k=wk, depth=PF)
                c0, c1 = MK(inner=reg, **kw), MK(inner=ring, **kw)
                if not (skg.skinny_gemm_check_config(M, K, N, c0)
                        and skg.skinny_gemm_check_config(M, K, N, c1)):
                    continue
                want = gu.bits_of(skg.skinny_gemm_bf16_with_config(A, B, c0))
                got = gu.bits_of(skg.skinny_gemm_bf16_with_config(A, B, c1))
                torch.cuda.synchronize()
                assert np.array_equal(got, want), (M, K, N, c1)


def test_mid_repeated_calls_identical():
    torch = gu.torch_cuda()
    for (M, K, N) in ((48, 7168, 2112), (64, 1536, 24576), (33, 7168, 256)):
        A_bits = inputs.make_a(M, K, N)
        A, B = gu.operands(A_bits, gu.cached_b(K, N), K)
        ref = gu.bits_of(skg.skinny_gemm_bf16(A, B))
        outs = [skg.skinny_gemm_bf16(A, B) for _ in range(20)]
        torch.cuda.synchronize()
        for o in outs:
            assert np.array_equal(gu.bits_of(o), ref), (M, K, N)


@pytest.mark.parametrize("M", [17, 31, 48, 64])
def test_mid_edges(M):
    """K = 0 (zeros), K < 8 (one thread per output), K = 8, 9 (one window and
    a ragged one), N = 1 and 3, into a strided bf16 buffer whose padding
    columns stay untouched."""
    torch = gu.torch_cuda()
    for K in (0, 1, 7, 8, 9, 130):
        for N in (1, 3, 37):
            ld = max(8, gu.round8(K))
            A_bits = inputs.make_a(M, K, N, lda=ld)
            B_bits = inputs.make_b(K, N, ldb=ld)
            A, B = gu.operands(A_bits, B_bits, K)
            buf = torch.full((M, N + 5), float("nan"), dtype=torch.bfloat16, device="cuda")
            skg.skinny_gemm_bf16(A, B, out=buf[:, :N])
            torch.cuda.synchronize()
            if K == 0:
                assert np.all(gu.to_f64(buf[:, :N]) == 0.0), (M, K, N)
            else:
                r = gu.assess(buf[:, :N], A_bits, B_bits, K)
                assert r["ok"], (M, K, N, r)
            assert np.isnan(gu.to_f64(buf[:, N:])).all(), (M, K, N)


def test_two_streams_mid_tier_and_fp32_weights():
    """Split-K calls of the middle tier (one pass and two passes) and of the
    fp32-weight path on two streams at once: each stream has its own
    workspace, so every result equals its single-stream one."""
    torch = gu.torch_cuda()
    p1 = MK(inner=GA, split_k=4, row_tiles=1, waves_n=1, waves_k=2, depth=2)
    p2 = MK(backend=P2, inner=RG, split_k=6, row_tiles=1, waves_n=1, waves_k=1, depth=2)
    pf = MK(inner=skg.SKG_INNER_VALU, split_k=4, row_tiles=1, waves_n=1, waves_k=2, depth=4)
    A1, B1 = gu.operands(inputs.make_a(40, 7168, 2112), gu.cached_b(7168, 2112), 7168)
    A2, B2 = gu.operands(inputs.make_a(64, 7168, 256), gu.cached_b(7168, 256), 7168)
    A3b = inputs.make_a(12, 7168, 384)
    A3, W3 = gu.operands_f32w(A3b, inputs.make_w_f32(7168, 384), 7168)
    calls = [lambda s: skg.skinny_gemm_bf16_with_config(A1, B1, p1, stream=s),
             lambda s: skg.skinny_gemm_bf16_with_config(A2, B2, p2, stream=s),
             lambda s: skg.skinny_gemm_f32w_with_config(A3, W3, pf, stream=s)]
    ref = [gu.bits_of(c(None)) for c in calls]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for i in range(12):
        for j, c in enumerate(calls):
            s = streams[(i + j) % 2]
            with torch.cuda.stream(s):
                outs.append((j, c(s)))
    torch.cuda.synchronize()
    for j, o in outs:
        assert np.array_equal(gu.bits_of(o), ref[j]), j

"""HIP path vs the oracle, element by element (GPU).

* every point of the five decode workloads at full size, with the
  configuration the dispatch table picks (what bench.py times);
* every kernel variant forced through the explicit-config entry on shapes
  that span several row blocks and splits and end in ragged K and N tails.
"""
import numpy as np
import pytest

import oracle
import latency_decode_gemm_amd as skg
from latency_decode_gemm_amd import inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

MK = skg.SkgConfig.make
V, F, GA = skg.SKG_INNER_VALU, skg.SKG_INNER_MFMA, skg.SKG_INNER_MFMA_GA
VG = skg.SKG_INNER_VALU_GA
RF, RG = skg.SKG_INNER_MFMA_RING, skg.SKG_INNER_MFMA_RING_GA
SY, SH = skg.SKG_INNER_MFMA_RING_SYNC, skg.SKG_INNER_MFMA_RING_SHARED
P2 = skg.SKG_BACKEND_SPLITK_2PASS
EV = skg.SKG_BACKEND_EVEN


def _run_point(p):
    torch = gu.torch_cuda()
    M, K, N = p["M"], p["K"], p["N"]
    A_bits = inputs.make_a(M, K, N)
    B_bits = gu.cached_b(K, N)
    A, B = gu.operands(A_bits, B_bits, K)
    if p["out"] == "bf16":
        ldc = p["ldc"] or N
        buf = torch.full((M, ldc), float("nan"), dtype=torch.bfloat16, device="cuda")
        C = buf[:, :N]
    else:
        buf = None
        C = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    skg.skinny_gemm_bf16(A, B, out=C)
    torch.cuda.synchronize()
    return A_bits, B_bits, C, buf


@pytest.mark.parametrize("p", inputs.all_points(),
                         ids=lambda p: f"M{p['M']}_K{p['K']}_N{p['N']}_{p['out']}"
                                       + (f"_ldc{p['ldc']}" if p["ldc"] else ""))
def test_workload_point(p):
    A_bits, B_bits, C, buf = _run_point(p)
    r = gu.assess(C, A_bits, B_bits, p["K"])
    assert r["ok"], r
    if buf is not None and buf.shape[1] > p["N"]:
        # columns [N, ldc) of the strided output are untouched (still NaN)
        assert np.isnan(gu.to_f64(buf[:, p["N"]:])).all()


SHAPES = [(1, 2880, 200), (3, 1003, 77), (8, 4104, 130), (16, 2880, 128), (16, 777, 33),
          (5, 7168, 100), (11, 520, 50), (2, 9, 5), (13, 33, 300)]


def _configs():
    out = []
    for (R, PF) in skg._capi.VALU_VARIANTS:
        out += [MK(inner=V, split_k=1, row_tiles=R, waves_n=1, waves_k=1, depth=PF),
                MK(inner=V, split_k=1, row_tiles=R, waves_n=2, waves_k=3, depth=PF, rb_per_wg=3),
                MK(inner=V, split_k=3, row_tiles=R, waves_n=1, waves_k=2, depth=PF, rb_per_wg=2),
                MK(backend=P2, inner=V, split_k=2, row_tiles=R, waves_n=2, waves_k=1, depth=PF),
                MK(inner=VG, split_k=1, row_tiles=R, waves_n=1, waves_k=1, depth=PF),
                MK(inner=VG, split_k=1, row_tiles=R, waves_n=2, waves_k=3, depth=PF, rb_per_wg=3),
                MK(inner=VG, split_k=3, row_tiles=R, waves_n=1, waves_k=2, depth=PF, rb_per_wg=2),
                MK(backend=P2, inner=VG, split_k=2, row_tiles=R, waves_n=2, waves_k=1, depth=PF),
                MK(backend=EV, inner=V, split_k=1, row_tiles=R, waves_n=2, waves_k=2, depth=PF),
                MK(backend=EV, inner=VG, split_k=1, row_tiles=R, waves_n=1, waves_k=1, depth=PF),
                MK(backend=EV, inner=V, split_k=2, row_tiles=R, waves_n=2, waves_k=1, depth=PF),
                MK(backend=EV, inner=VG, split_k=4, row_tiles=R, waves_n=1, waves_k=2, depth=PF,
                   rb_per_wg=3)]
    for (G, PF) in skg._capi.MFMA_VARIANTS:
        out += [MK(inner=F, split_k=1, row_tiles=G, waves_n=1, waves_k=1, depth=PF),
                # 8 waves of 4 transpose tiles each would not leave LDS for A
                MK(inner=F, split_k=1, row_tiles=G, waves_n=2, waves_k=4 if G < 4 else 2, depth=PF),
                MK(inner=F, split_k=2, row_tiles=G, waves_n=1, waves_k=3, depth=PF, rb_per_wg=2),
                MK(inner=GA, split_k=1, row_tiles=G, waves_n=1, waves_k=1, depth=PF),
                MK(inner=GA, split_k=1, row_tiles=G, waves_n=2, waves_k=2, depth=PF, rb_per_wg=3),
                MK(inner=GA, split_k=3, row_tiles=G, waves_n=1, waves_k=2, depth=PF),
                MK(backend=P2, inner=GA, split_k=4, row_tiles=G, waves_n=1, waves_k=1, depth=PF,
                   rb_per_wg=2),
                MK(backend=P2, inner=F, split_k=2, row_tiles=G, waves_n=1, waves_k=2, depth=PF),
                MK(inner=RF, split_k=1, row_tiles=G, waves_n=1, waves_k=1, depth=PF),
                MK(inner=RF, split_k=2, row_tiles=G, waves_n=1, waves_k=2, depth=PF, rb_per_wg=2),
                MK(inner=RG, split_k=1, row_tiles=G, waves_n=2, waves_k=1, depth=PF, rb_per_wg=3),
                MK(inner=RG, split_k=3, row_tiles=G, waves_n=1, waves_k=2, depth=PF),
                MK(backend=P2, inner=RG, split_k=2, row_tiles=G, waves_n=1, waves_k=1, depth=PF),
                MK(backend=EV, inner=GA, split_k=1, row_tiles=G, waves_n=1, waves_k=2, depth=PF),
                MK(backend=EV, inner=F, split_k=1, row_tiles=G, waves_n=2, waves_k=1, depth=PF),
                MK(backend=EV, inner=RG, split_k=1, row_tiles=G, waves_n=1, waves_k=1, depth=PF),
                MK(backend=EV, inner=GA, split_k=2, row_tiles=G, waves_n=1, waves_k=2, depth=PF),
                MK(backend=EV, inner=RG, split_k=4, row_tiles=G, waves_n=1, waves_k=1, depth=PF),
                MK(backend=EV, inner=RF, split_k=4, row_tiles=G, waves_n=1, waves_k=1, depth=PF,
                   rb_per_wg=2)]
    # the barrier kinds: several waves on one K range (direct stores), K-wave
    # groups (the stash; one K-wave where two do not fit the LDS with a deep
    # ring), a one-pass and a two-pass split, rows dealt evenly
    for (G, PF) in skg._capi.SYNC_VARIANTS:
        for inner in (SY, SH):
            if inner == SH and (G, PF) not in skg._capi.SHARED_VARIANTS:
                continue
            wk = 2 if _fits_a_shape(MK(inner=inner, split_k=1, row_tiles=G, waves_n=2,
                                       waves_k=2, depth=PF)) else 1
            out += [MK(inner=inner, split_k=1, row_tiles=G, waves_n=3, waves_k=1, depth=PF,
                       rb_per_wg=2),
                    MK(inner=inner, split_k=1, row_tiles=G, waves_n=2, waves_k=wk, depth=PF),
                    MK(inner=inner, split_k=3, row_tiles=G, waves_n=2, waves_k=1, depth=PF),
                    MK(backend=P2, inner=inner, split_k=2, row_tiles=G, waves_n=2, waves_k=1,
                       depth=PF),
                    MK(backend=EV, inner=inner, split_k=1, row_tiles=G, waves_n=2, waves_k=wk,
                       depth=PF)]
    return out


def _fits_a_shape(cfg):
    return any(skg.skinny_gemm_check_config(M, K, N, cfg) for (M, K, N) in SHAPES)



def _cfg_id(c):
    return ("p2_" if c.backend == P2 else "ev_" if c.backend == EV else "") + \
        {V: "valu", F: "mfma", GA: "mfmaga", VG: "valuga", RF: "ring", RG: "ringga",
         SY: "ringsync", SH: "ringshared"}[c.inner] + \
        f"_S{c.split_k}_r{c.row_tiles}_n{c.waves_n}_k{c.waves_k}_d{c.depth}_b{c.rb_per_wg}"


@pytest.mark.parametrize("cfg", _configs(), ids=_cfg_id)
def test_forced_config(cfg):
    torch = gu.torch_cuda()
    ran = 0
    for (M, K, N) in SHAPES:
        ld = gu.round8(K)
        A_bits = inputs.make_a(M, K, N, lda=ld)
        B_bits = inputs.make_b(K, N, ldb=ld)
        A, B = gu.operands(A_bits, B_bits, K)
        for out_dtype in (torch.float32, torch.bfloat16):
            if not skg.skinny_gemm_check_config(M, K, N, cfg):
                with pytest.raises(skg.SkinnyGemmError):
                    skg.skinny_gemm_bf16_with_config(A, B, cfg, out_dtype=out_dtype)
                continue
            C = skg.skinny_gemm_bf16_with_config(A, B, cfg, out_dtype=out_dtype)
            torch.cuda.synchronize()
            r = gu.assess(C, A_bits, B_bits, K)
            assert r["ok"], (M, K, N, out_dtype, r)
            ran += 1
    assert ran > 0


@pytest.mark.parametrize("variant", list(skg._capi.MFMA_VARIANTS), ids=lambda v: f"G{v[0]}_d{v[1]}")
def test_lds_ring_equals_register_ring(variant):
    """The LDS-ring MFMA kernels issue the same MFMAs on the same operands in
    the same order as the register-ring ones, so outputs agree bit for bit,
    K tails, ragged N, every M and split-K included."""
    torch = gu.torch_cuda()
    G, PF = variant
    ran = 0
    for (M, K, N) in [(16, 1000, 333), (1, 2880, 200), (7, 136, 1000), (13, 8, 19), (16, 4104, 130)]:
        ld = gu.round8(K)
        A_bits = inputs.make_a(M, K, N, lda=ld)
        B_bits = inputs.make_b(K, N, ldb=ld)
        A, B = gu.operands(A_bits, B_bits, K)
        for (reg, ring) in ((F, RF), (GA, RG)):
            for (be, S, wn, wk, rpw) in ((0, 1, 1, 1, 1), (0, 1, 2, 2, 2), (1, 2, 1, 2, 1),
                                         (P2, 3, 2, 1, 1)):
                kw = dict(split_k=S, row_tiles=G, waves_n=wn, waves_k=wk, depth=PF, rb_per_wg=rpw)
                c0 = MK(backend=be, inner=reg, **kw) if be else MK(inner=reg, **kw)
                c1 = MK(backend=be, inner=ring, **kw) if be else MK(inner=ring, **kw)
                if not (skg.skinny_gemm_check_config(M, K, N, c0)
                        and skg.skinny_gemm_check_config(M, K, N, c1)):
                    continue
                want = gu.bits_of(skg.skinny_gemm_bf16_with_config(A, B, c0))
                out = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
                skg.skinny_gemm_bf16_with_config(A, B, c1, out=out)
                torch.cuda.synchronize()
                assert np.array_equal(gu.bits_of(out), want), (M, K, N, c1)
                ran += 1
    assert ran >= 8


@pytest.mark.parametrize("variant", list(skg._capi.VALU_VARIANTS),
                         ids=lambda v: f"r{v[0]}_d{v[1]}")
def test_every_valu_instantiation(variant):
    """Each compiled (M, row_tiles, depth) VALU kernel, once."""
    torch = gu.torch_cuda()
    R, PF = variant
    K, N = 1021, 37
    ld = gu.round8(K)
    B_bits = inputs.make_b(K, N, ldb=ld)
    for M in range(1, 17):
        A_bits = inputs.make_a(M, K, N, lda=ld)
        A, B = gu.operands(A_bits, B_bits, K)
        cfg = MK(inner=V, split_k=1, row_tiles=R, waves_n=1, waves_k=2, depth=PF)
        C = skg.skinny_gemm_bf16_with_config(A, B, cfg)
        torch.cuda.synchronize()
        r = gu.assess(C, A_bits, B_bits, K)
        assert r["ok"], (M, r)


def test_default_dispatch_on_small_grid():
    torch = gu.torch_cuda()
    for M in (1, 2, 4, 7, 8, 9, 12, 16):
        for (K, N) in ((64, 16), (300, 45), (2048, 256), (2056, 96)):
            ld = gu.round8(K)
            A_bits = inputs.make_a(M, K, N, lda=ld)
            B_bits = inputs.make_b(K, N, ldb=ld)
            A, B = gu.operands(A_bits, B_bits, K)
            C = skg.skinny_gemm_bf16(A, B)
            torch.cuda.synchronize()
            r = gu.assess(C, A_bits, B_bits, K)
            assert r["ok"], (M, K, N, r)

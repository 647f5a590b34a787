"""The no-allocation entry point (GPU): skinny_gemm_bf16_noalloc, whose
split-K workspace is the library's static per-GPU scratch, called through
the C ABI.  Its output equals skinny_gemm_bf16's bit for bit (same
configuration, same kernels, same summation order) and matches the oracle,
on two calls in a row, the second with a smaller input, for shapes whose
configuration splits K (the scratch is used) and one that does not."""
import ctypes

import numpy as np
import pytest

import latency_decode_gemm_amd as skg
from latency_decode_gemm_amd import _capi, inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _noalloc(A, B, out, stream):
    """Through the C ABI directly (the Python wrapper only marshals these)."""
    torch = gu.torch_cuda()
    M, K = A.shape
    N = B.shape[0]
    odt = skg.SKG_OUT_BF16 if out.dtype == torch.bfloat16 else skg.SKG_OUT_F32
    st = _capi.lib().skinny_gemm_bf16_noalloc(
        A.data_ptr(), B.data_ptr(), out.data_ptr(), M, N, K, A.stride(0), B.stride(0),
        out.stride(0), odt, ctypes.c_void_p(stream.cuda_stream))
    assert st == skg.SKG_OK, skg.skinny_gemm_strerror(st)


# (first call, second call with a smaller input): M, K, N, output dtype, ldc
PAIRS = [
    # router points with a single-pass K split (4 then 4 splits, 2 then 2)
    ((16, 7168, 384, "f32", None), (16, 7168, 256, "f32", None)),
    ((8, 7168, 384, "f32", None), (5, 7168, 256, "f32", None)),
    # split 4 (M = 16) then split 2 (M = 8): another geometry in the same scratch
    ((16, 7168, 256, "f32", None), (8, 7168, 256, "f32", None)),
    # middle-tier splits (two token tiles, 4 splits)
    ((32, 7168, 384, "f32", None), (24, 7168, 256, "f32", None)),
    # qkv_a-style, bf16 into a strided buffer: a 3-way split, then none (the
    # scratch is not touched)
    ((16, 7168, 2112, "bf16", 4096), (3, 7168, 2112, "bf16", 4096)),
]


@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: "M%d_N%d_then_M%d_N%d" % (
    p[0][0], p[0][2], p[1][0], p[1][2]))
def test_noalloc_matches_allocating_entry_and_oracle(pair):
    torch = gu.torch_cuda()
    s = torch.cuda.Stream()
    for (M, K, N, out, ldc) in pair:
        cfg = skg.skinny_gemm_dispatch(M, K, N)
        print(f"noalloc M={M} K={K} N={N} cfg={cfg.as_tuple()}", flush=True)
        assert (skg.skinny_gemm_workspace_bytes(M, K, N, cfg)
                <= skg.SKG_SCRATCH_PARTIAL_BYTES + skg.SKG_SCRATCH_SLOT_BYTES)
        A_bits = inputs.make_a(M, K, N)
        B_bits = gu.cached_b(K, N)
        A, B = gu.operands(A_bits, B_bits, K)
        dt = torch.bfloat16 if out == "bf16" else torch.float32
        buf = torch.full((M, ldc or N), float("nan"), dtype=dt, device="cuda")
        ref = torch.full((M, ldc or N), float("nan"), dtype=dt, device="cuda")
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            _noalloc(A, B, buf[:, :N], s)
            skg.skinny_gemm_bf16(A, B, out=ref[:, :N], stream=s)
        torch.cuda.synchronize()
        assert np.array_equal(gu.bits_of(buf), gu.bits_of(ref)), (M, K, N)
        r = gu.assess(buf[:, :N], A_bits, B_bits, K)
        assert r["ok"], (M, K, N, r)
        if ldc and ldc > N:
            assert np.isnan(gu.to_f64(buf[:, N:])).all()


def test_noalloc_repeated_calls_identical():
    """Back-to-back split-K calls on one stream share the scratch: each one
    leaves its tree slots empty for the next, so 500 calls in a row give the
    first call's bits."""
    torch = gu.torch_cuda()
    M, K, N = 16, 7168, 256
    assert skg.skinny_gemm_dispatch(M, K, N).split_k > 1
    A, B = gu.operands(inputs.make_a(M, K, N), gu.cached_b(K, N), K)
    s = torch.cuda.Stream()
    ref = torch.empty((M, N), dtype=torch.float32, device="cuda")
    outs = [torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
            for _ in range(50)]
    with torch.cuda.stream(s):
        skg.skinny_gemm_bf16(A, B, out=ref, stream=s)
    torch.cuda.synchronize()
    for rnd in range(10):
        with torch.cuda.stream(s):
            for o in outs:
                _noalloc(A, B, o, s)
        torch.cuda.synchronize()
        for i, o in enumerate(outs):
            assert torch.equal(o.view(torch.int32), ref.view(torch.int32)), (rnd, i)


def test_noalloc_rejects_a_workspace_beyond_the_scratch():
    """The two-pass split of qkv_a-style M = 64 needs more partials than the
    scratch holds: SKG_ERR_SCRATCH_TOO_SMALL, and the output is untouched."""
    torch = gu.torch_cuda()
    M, K, N = 64, 7168, 2112
    cfg = skg.skinny_gemm_dispatch(M, K, N)
    assert cfg.backend == skg.SKG_BACKEND_SPLITK_2PASS, cfg
    assert skg.skinny_gemm_workspace_bytes(M, K, N, cfg) > skg.SKG_SCRATCH_PARTIAL_BYTES
    A = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((N, K), dtype=torch.bfloat16, device="cuda")
    out = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    with pytest.raises(skg.SkinnyGemmError) as e:
        skg.skinny_gemm_bf16_noalloc(A, B, out)
    assert e.value.status == skg.SKG_ERR_SCRATCH_TOO_SMALL
    torch.cuda.synchronize()
    assert torch.isnan(out).all()

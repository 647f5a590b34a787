"""Edge cases on the GPU: degenerate sizes, ragged K and N, padded and
strided layouts, the bytes outside C, and error returns."""
import numpy as np
import pytest

import latency_decode_gemm_amd as skg
from latency_decode_gemm_amd import inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

MK = skg.SkgConfig.make
V, F = skg.SKG_INNER_VALU, skg.SKG_INNER_MFMA
SENT_BF16 = 0x7FC1
SENT_F32 = 0x7FC00001


def _sentinel(M, ldc, bf16):
    torch = gu.torch_cuda()
    if bf16:
        t = torch.full((M, ldc), SENT_BF16, dtype=torch.int16, device="cuda")
        return t.view(torch.bfloat16)
    t = torch.full((M, ldc), SENT_F32, dtype=torch.int32, device="cuda")
    return t.view(torch.float32)


CFGS = [None,
        MK(inner=V, split_k=2, row_tiles=1, waves_n=1, waves_k=2, depth=4),
        MK(inner=F, split_k=1, row_tiles=1, waves_n=1, waves_k=2, depth=4),
        MK(inner=F, split_k=3, row_tiles=1, waves_n=2, waves_k=1, depth=2),
        MK(inner=skg.SKG_INNER_MFMA_GA, split_k=1, row_tiles=2, waves_n=1, waves_k=3, depth=2,
           rb_per_wg=2)]


def _call(A, B, cfg, out):
    if cfg is None:
        return skg.skinny_gemm_bf16(A, B, out=out)
    return skg.skinny_gemm_bf16_with_config(A, B, cfg, out=out)


def test_ragged_k_sweep():
    torch = gu.torch_cuda()
    Ks = list(range(1, 41)) + [127, 128, 129, 255, 256, 257, 1023, 1025, 2047, 2049]
    N = 19
    for K in Ks:
        ld = gu.round8(K)
        B_bits = inputs.make_b(K, N, ldb=ld)
        for M in (1, 5, 16):
            A_bits = inputs.make_a(M, K, N, lda=ld)
            A, B = gu.operands(A_bits, B_bits, K)
            for cfg in CFGS:
                if cfg is not None and not skg.skinny_gemm_check_config(M, K, N, cfg):
                    continue
                C = _call(A, B, cfg, None)
                torch.cuda.synchronize()
                r = gu.assess(C, A_bits, B_bits, K)
                assert r["ok"], (K, M, cfg, r)


def test_ragged_n_sweep():
    torch = gu.torch_cuda()
    K = 264
    for N in (1, 2, 3, 4, 5, 15, 16, 17, 31, 63, 65, 127, 129):
        B_bits = inputs.make_b(K, N)
        for M in (1, 3, 9, 16):
            A_bits = inputs.make_a(M, K, N)
            A, B = gu.operands(A_bits, B_bits, K)
            for cfg in CFGS:
                if cfg is not None and not skg.skinny_gemm_check_config(M, K, N, cfg):
                    continue
                C = _call(A, B, cfg, None)
                torch.cuda.synchronize()
                r = gu.assess(C, A_bits, B_bits, K)
                assert r["ok"], (N, M, cfg, r)


@pytest.mark.parametrize("bf16", [True, False], ids=["bf16", "f32"])
def test_strided_output_leaves_padding(bf16):
    torch = gu.torch_cuda()
    M, K, N, ldc = 7, 1000, 100, 160
    A_bits = inputs.make_a(M, K, N)
    B_bits = inputs.make_b(K, N)
    A, B = gu.operands(A_bits, B_bits, K)
    for cfg in CFGS:
        if cfg is not None and not skg.skinny_gemm_check_config(M, K, N, cfg):
            continue
        buf = _sentinel(M, ldc, bf16)
        C = buf[:, :N]
        _call(A, B, cfg, C)
        torch.cuda.synchronize()
        raw = gu.bits_of(buf)
        sent = SENT_BF16 if bf16 else SENT_F32
        assert np.all(raw[:, N:] == sent)
        r = gu.assess(C, A_bits, B_bits, K)
        assert r["ok"], (cfg, r)


def test_qkv_a_strided_sentinel_full_size():
    """The qkv_a-style point: bf16 into a [M, 4096] buffer, columns >= 2112 kept."""
    torch = gu.torch_cuda()
    K, N, ldc = 7168, 2112, 4096
    B_bits = gu.cached_b(K, N)
    for M in (2, 3, 8, 16):
        A_bits = inputs.make_a(M, K, N)
        A, B = gu.operands(A_bits, B_bits, K)
        buf = _sentinel(M, ldc, True)
        skg.skinny_gemm_bf16(A, B, out=buf[:, :N])
        torch.cuda.synchronize()
        raw = gu.bits_of(buf)
        assert np.all(raw[:, N:] == SENT_BF16)
        r = gu.assess(buf[:, :N], A_bits, B_bits, K)
        assert r["ok"], (M, r)


def test_padded_leading_dimensions_are_not_read():
    """lda, ldb > K with NaN in the padding: the result stays finite and correct."""
    torch = gu.torch_cuda()
    M, K, N = 6, 1000, 70
    A_bits = inputs.make_a(M, K, N, lda=1024)
    B_bits = inputs.make_b(K, N, ldb=1096)
    A, B = gu.operands(A_bits, B_bits, K)
    for cfg in CFGS:
        if cfg is not None and not skg.skinny_gemm_check_config(M, K, N, cfg):
            continue
        C = _call(A, B, cfg, None)
        torch.cuda.synchronize()
        r = gu.assess(C, A_bits, B_bits, K)
        assert r["ok"], (cfg, r)


def test_empty_and_zero_k():
    torch = gu.torch_cuda()
    # M = 0 and N = 0: nothing written
    B = gu.to_dev(inputs.make_b(64, 8))
    A0 = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    C0 = torch.empty((0, 8), dtype=torch.float32, device="cuda")
    skg.skinny_gemm_bf16(A0, B, out=C0)
    A = gu.to_dev(inputs.make_a(3, 64, 8))
    B0 = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    buf = _sentinel(3, 8, False)
    skg.skinny_gemm_bf16(A, B0, out=buf[:, :0])
    torch.cuda.synchronize()
    assert np.all(gu.bits_of(buf) == SENT_F32)
    # K = 0: zeros, padding untouched
    for bf16 in (True, False):
        buf = _sentinel(4, 24, bf16)
        Ae = torch.empty((4, 0), dtype=torch.bfloat16, device="cuda")
        Be = torch.empty((20, 0), dtype=torch.bfloat16, device="cuda")
        skg.skinny_gemm_bf16(Ae, Be, out=buf[:, :20])
        torch.cuda.synchronize()
        raw = gu.bits_of(buf)
        assert np.all(raw[:, :20] == 0)
        assert np.all(raw[:, 20:] == (SENT_BF16 if bf16 else SENT_F32))


def test_maximum_m_and_large_n():
    torch = gu.torch_cuda()
    M, K, N = 16, 2048, 40000
    A_bits = inputs.make_a(M, K, N)
    B_bits = inputs.make_b(K, N)
    A, B = gu.operands(A_bits, B_bits, K)
    C = skg.skinny_gemm_bf16(A, B, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    r = gu.assess(C, A_bits, B_bits, K)
    assert r["ok"], r


@pytest.mark.parametrize("shape, cfg", [
    ((16, 65536, 384), None),              # long K through the default rule
    ((4, 64, 1 << 20), None),              # a million rows of B, tiny K
    ((16, 1536, 98304), dict(inner=skg.SKG_INNER_MFMA_RING_GA, split_k=1, row_tiles=1,
                             waves_n=3, waves_k=1, depth=3, rb_per_wg=2)),  # 302 MB of B
], ids=["longK", "millionN", "ring302MB"])
def test_large_shapes(shape, cfg):
    torch = gu.torch_cuda()
    M, K, N = shape
    A_bits = inputs.make_a(M, K, N)
    B_bits = inputs.make_b(K, N)
    A, B = gu.operands(A_bits, B_bits, K)
    if cfg is None:
        C = skg.skinny_gemm_bf16(A, B, out_dtype=torch.bfloat16)
    else:
        C = skg.skinny_gemm_bf16_with_config(A, B, skg.SkgConfig.make(**cfg),
                                             out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    r = gu.assess(C, A_bits, B_bits, K)
    assert r["ok"], r


def test_error_returns():
    torch = gu.torch_cuda()
    A65 = torch.zeros((65, 64), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((8, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(skg.SkinnyGemmError) as e:
        skg.skinny_gemm_bf16(A65, B)
    assert e.value.status == skg.SKG_ERR_UNSUPPORTED
    # over fp32 weights the VALU kernels take at most 16 tokens
    with pytest.raises(skg.SkinnyGemmError) as e:
        skg.skinny_gemm_f32w(A65[:17], torch.zeros((8, 64), dtype=torch.float32, device="cuda"))
    assert e.value.status == skg.SKG_ERR_UNSUPPORTED
    # A offset by one element: not 16-byte aligned
    base = torch.zeros((4, 72), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(skg.SkinnyGemmError) as e:
        skg.skinny_gemm_bf16(base[:, 1:65], B)
    assert e.value.status == skg.SKG_ERR_MISALIGNED
    # lda = 9 (not a multiple of 8)
    A9 = torch.zeros((4, 9), dtype=torch.bfloat16, device="cuda")
    B9 = torch.zeros((8, 9), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(skg.SkinnyGemmError) as e:
        skg.skinny_gemm_bf16(A9, B9)
    assert e.value.status == skg.SKG_ERR_MISALIGNED
    with pytest.raises(TypeError):
        skg.skinny_gemm_bf16(A9.float(), B9)


def test_stream_read_probe_folds_every_word():
    """The read-ceiling probe touches every 16-byte word exactly once: the XOR
    of its per-workgroup words equals the XOR of the buffer; bad arguments are
    rejected before any launch."""
    torch = gu.torch_cuda()
    rng = np.random.default_rng(11)
    for nbytes in (16, 4096 + 48, (1 << 20) + 16 * 37, 3 << 22):
        host = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
        src = torch.from_numpy(host.view(np.int32)).cuda()
        sink = torch.zeros(512, dtype=torch.int32, device="cuda")
        skg.skinny_gemm_stream_read(src, sink)
        torch.cuda.synchronize()
        got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
        assert got == np.bitwise_xor.reduce(host), nbytes
    lib = skg._capi.lib()
    src = torch.zeros(64, dtype=torch.int32, device="cuda")
    sink = torch.zeros(512, dtype=torch.int32, device="cuda")
    assert lib.skinny_gemm_stream_read(src.data_ptr() + 4, 16, sink.data_ptr(), None) == \
        skg.SKG_ERR_MISALIGNED
    assert lib.skinny_gemm_stream_read(src.data_ptr(), 24, sink.data_ptr(), None) == \
        skg.SKG_ERR_MISALIGNED
    assert lib.skinny_gemm_stream_read(src.data_ptr(), 16, None, None) == skg.SKG_ERR_INVALID_ARG
    assert lib.skinny_gemm_stream_read(None, 0, None, None) == skg.SKG_OK


def test_capture_before_warmup_reports_not_warmed():
    """A split-K call captured on a stream whose workspace was never sized
    returns SKG_ERR_NOT_WARMED (nothing is allocated or launched while
    capturing); after skinny_gemm_warmup on that stream the same capture
    works and its replay equals the eager result."""
    torch = gu.torch_cuda()
    M, K, N = 16, 7168, 256
    cfg = skg.SkgConfig.make(inner=skg.SKG_INNER_MFMA_GA, split_k=4, row_tiles=1, waves_n=1,
                             waves_k=2, depth=2)
    A_bits = inputs.make_a(M, K, N)
    A, B = gu.operands(A_bits, gu.cached_b(K, N), K)
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        with pytest.raises(skg.SkinnyGemmError) as e:
            skg.skinny_gemm_bf16_with_config(A, B, cfg, out=out, stream=s)
    assert e.value.status == skg.SKG_ERR_NOT_WARMED
    del g
    # an eager call on the stream sizes its workspace; capture then works
    with torch.cuda.stream(s):
        want = gu.bits_of(skg.skinny_gemm_bf16_with_config(A, B, cfg, stream=s))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        skg.skinny_gemm_bf16_with_config(A, B, cfg, out=out, stream=s)
    out.fill_(float("nan"))
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    assert np.array_equal(gu.bits_of(out), want)


def test_graph_survives_workspace_growth():
    """A graph captured after a small warm-up keeps working after a larger
    split-K shape grows the same stream's workspace: the replaced workspace
    stays allocated (the graph's kernels still address it), so every replay
    still matches the oracle and the eager result, with eager calls on the
    grown workspace between the replays."""
    torch = gu.torch_cuda()
    K = 7168
    small, large = (8, 256), (16, 384)  # router points: split 2, then split 4
    c_small = skg.skinny_gemm_dispatch(small[0], K, small[1])
    c_large = skg.skinny_gemm_dispatch(large[0], K, large[1])
    assert c_small.split_k > 1 and c_large.split_k > 1
    assert (skg.skinny_gemm_workspace_bytes(large[0], K, large[1], c_large)
            > skg.skinny_gemm_workspace_bytes(small[0], K, small[1], c_small))
    s = torch.cuda.Stream()
    probs = {}
    for (M, N) in (small, large):
        A_bits = inputs.make_a(M, K, N)
        B_bits = gu.cached_b(K, N)
        probs[(M, N)] = (A_bits, B_bits) + gu.operands(A_bits, B_bits, K)
    # a fresh stream: the small warm-up sizes its workspace for the small
    # shape only
    with torch.cuda.stream(s):
        skg.skinny_gemm_warmup([(K, small[1])], [small[0]], stream=s)
    A_bits, B_bits, A, B = probs[small]
    out = torch.empty(small, dtype=torch.float32, device="cuda")
    with torch.cuda.stream(s):
        want = gu.bits_of(skg.skinny_gemm_bf16(A, B, stream=s))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        skg.skinny_gemm_bf16(A, B, out=out, stream=s)
    # grow the workspace of the same stream (the old one is retired, not freed)
    with torch.cuda.stream(s):
        skg.skinny_gemm_warmup([(K, large[1])], [large[0]], stream=s)
    La_bits, Lb_bits, LA, LB = probs[large]
    for i in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        r = gu.assess(out, A_bits, B_bits, K)
        assert r["ok"], (i, r)
        assert np.array_equal(gu.bits_of(out), want), i
        # eager work on the grown workspace between the replays, on the same stream
        with torch.cuda.stream(s):
            big = skg.skinny_gemm_bf16(LA, LB, stream=s)
        torch.cuda.synchronize()
        r = gu.assess(big, La_bits, Lb_bits, K)
        assert r["ok"], (i, r)

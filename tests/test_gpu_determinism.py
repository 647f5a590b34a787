"""Bit-reproducibility on the GPU: repeated calls, default vs explicit
configuration, warm-up, concurrent streams, and HIP graph replay."""
import numpy as np
import pytest

import latency_decode_gemm_amd as skg
from latency_decode_gemm_amd import inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

MK = skg.SkgConfig.make


def _problem(M, K, N):
    A_bits = inputs.make_a(M, K, N)
    B_bits = gu.cached_b(K, N)
    return gu.operands(A_bits, B_bits, K)


@pytest.mark.parametrize("shape", [(16, 7168, 256), (4, 7168, 384), (8, 14336, 7168),
                                   (16, 1536, 24576), (1, 2880, 128)],
                         ids=lambda s: "M%d_K%d_N%d" % s)
def test_repeated_calls_identical(shape):
    torch = gu.torch_cuda()
    A, B = _problem(*shape)
    ref = gu.bits_of(skg.skinny_gemm_bf16(A, B))
    outs = [skg.skinny_gemm_bf16(A, B) for _ in range(50)]
    torch.cuda.synchronize()
    for o in outs:
        assert np.array_equal(gu.bits_of(o), ref)


def test_default_equals_explicit_dispatch_config():
    torch = gu.torch_cuda()
    for p in inputs.all_points():
        A, B = _problem(p["M"], p["K"], p["N"])
        cfg = skg.skinny_gemm_dispatch(p["M"], p["K"], p["N"])
        c1 = skg.skinny_gemm_bf16(A, B)
        c2 = skg.skinny_gemm_bf16_with_config(A, B, cfg)
        torch.cuda.synchronize()
        assert np.array_equal(gu.bits_of(c1), gu.bits_of(c2)), p


def test_split_k_forced_is_reproducible():
    torch = gu.torch_cuda()
    cases = [(16, MK(inner=skg.SKG_INNER_MFMA, split_k=4, row_tiles=1, waves_n=1, waves_k=2,
                     depth=2)),
             (16, MK(backend=skg.SKG_BACKEND_SPLITK_2PASS, inner=skg.SKG_INNER_MFMA_GA, split_k=4,
                     row_tiles=1, waves_n=1, waves_k=2, depth=2)),
             (16, MK(inner=skg.SKG_INNER_VALU, split_k=7, row_tiles=1, waves_n=1, waves_k=2,
                     depth=4)),
             (8, MK(inner=skg.SKG_INNER_VALU_GA, split_k=3, row_tiles=2, waves_n=1, waves_k=2,
                    depth=2)),
             # rows dealt evenly to 64 row blocks x 4 K slices
             (16, MK(backend=skg.SKG_BACKEND_EVEN, inner=skg.SKG_INNER_MFMA_RING_GA, split_k=4,
                     row_tiles=1, waves_n=1, waves_k=2, depth=2)),
             (4, MK(backend=skg.SKG_BACKEND_EVEN, inner=skg.SKG_INNER_VALU, split_k=2,
                    row_tiles=1, waves_n=1, waves_k=1, depth=4))]
    for M, cfg in cases:
        A, B = _problem(M, 7168, 256)
        _repeat_identical(lambda out: skg.skinny_gemm_bf16_with_config(A, B, cfg, out=out),
                          M, 256, 1000, (M, cfg))


def test_shared_activation_ring_repeats():
    """The shared activation ring hands each step's tile from the loading
    wave to the others across the step barrier; 1000 calls of it (several
    waves on one K range, and two K-wave groups with a one-pass split) are
    bit-identical to the first, which the float64 check also accepts."""
    SH = skg.SKG_INNER_MFMA_RING_SHARED
    cases = [(16, 1536, 3072, MK(inner=SH, split_k=1, row_tiles=1, waves_n=3, waves_k=1,
                                 depth=3, rb_per_wg=2)),
             (16, 7168, 256, MK(inner=SH, split_k=3, row_tiles=1, waves_n=2, waves_k=4,
                                depth=3))]
    for M, K, N, cfg in cases:
        A_bits = inputs.make_a(M, K, N)
        B_bits = inputs.make_b(K, N)
        A, B = gu.operands(A_bits, B_bits, K)
        first = skg.skinny_gemm_bf16_with_config(A, B, cfg)
        r = gu.assess(first, A_bits, B_bits, K)
        assert r["ok"], (cfg, r)
        _repeat_identical(lambda out: skg.skinny_gemm_bf16_with_config(A, B, cfg, out=out),
                          M, N, 1000, (M, K, N, cfg))


def _repeat_identical(call, M, N, reps, what, batch=50):
    """Runs call(out) reps times, batch outputs at a time, and stops at the
    first output that differs bit for bit from the first one."""
    torch = gu.torch_cuda()
    ref = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    call(ref)
    outs = [torch.empty((M, N), dtype=torch.float32, device="cuda") for _ in range(batch)]
    refi = ref.view(torch.int32)
    done = 0
    while done < reps:
        n = min(batch, reps - done)
        for o in outs[:n]:
            o.fill_(float("nan"))
        for o in outs[:n]:
            call(o)
        torch.cuda.synchronize()
        for i, o in enumerate(outs[:n]):
            assert torch.equal(o.view(torch.int32), refi), (what, "call", done + i + 1)
        done += n


@pytest.mark.parametrize("M", [8, 16])
@pytest.mark.parametrize("N", [256, 384])
def test_router_split_k_thousands_of_calls(M, N):
    """The router points that dispatch a single-pass K split (the partials
    combined along the exchange tree): 2000 calls, every one bit-identical to
    the first."""
    A, B = _problem(M, 7168, N)
    cfg = skg.skinny_gemm_dispatch(M, 7168, N)
    assert cfg.split_k > 1 and cfg.backend != skg.SKG_BACKEND_SPLITK_2PASS, cfg
    _repeat_identical(lambda out: skg.skinny_gemm_bf16(A, B, out=out), M, N, 2000, (M, N, cfg))


def test_warmup_then_same_bits():
    torch = gu.torch_cuda()
    shapes = [(7168, 256), (7168, 384), (2880, 128)]
    ms = [1, 2, 3, 4, 8, 16]
    A, B = _problem(16, 7168, 384)
    before = gu.bits_of(skg.skinny_gemm_bf16(A, B))
    n = skg.skinny_gemm_warmup(shapes, ms)
    assert n == len(skg.skinny_gemm_warmup_keys(shapes, ms))
    assert skg.skinny_gemm_warmup(shapes, ms) == n  # idempotent
    after = gu.bits_of(skg.skinny_gemm_bf16(A, B))
    torch.cuda.synchronize()
    assert np.array_equal(before, after)


def test_two_streams_concurrently():
    torch = gu.torch_cuda()
    A1, B1 = _problem(16, 7168, 256)
    A2, B2 = _problem(8, 7168, 384)
    cfg = MK(inner=skg.SKG_INNER_MFMA, split_k=4, row_tiles=1, waves_n=1, waves_k=2, depth=2)
    r1 = gu.bits_of(skg.skinny_gemm_bf16_with_config(A1, B1, cfg))
    r2 = gu.bits_of(skg.skinny_gemm_bf16_with_config(A2, B2, cfg))
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    outs1, outs2 = [], []
    for _ in range(20):
        with torch.cuda.stream(s1):
            outs1.append(skg.skinny_gemm_bf16_with_config(A1, B1, cfg, stream=s1))
        with torch.cuda.stream(s2):
            outs2.append(skg.skinny_gemm_bf16_with_config(A2, B2, cfg, stream=s2))
    torch.cuda.synchronize()
    for o in outs1:
        assert np.array_equal(gu.bits_of(o), r1)
    for o in outs2:
        assert np.array_equal(gu.bits_of(o), r2)


def test_graph_capture_replay():
    """Captured after warm-up; replayed several times with eager work between;
    every replay equals the eager result."""
    torch = gu.torch_cuda()
    shapes = [(7168, 256), (14336, 7168)]
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        skg.skinny_gemm_warmup(shapes, [1, 16], stream=s)
    A1, B1 = _problem(16, 7168, 256)
    A2, B2 = _problem(1, 14336, 7168)
    e1 = gu.bits_of(skg.skinny_gemm_bf16(A1, B1))
    e2 = gu.bits_of(skg.skinny_gemm_bf16(A2, B2, out_dtype=torch.bfloat16))
    out1 = torch.empty((16, 256), dtype=torch.float32, device="cuda")
    out2 = torch.empty((1, 7168), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        skg.skinny_gemm_bf16(A1, B1, out=out1, stream=s)
        skg.skinny_gemm_bf16(A2, B2, out=out2, stream=s)
    for i in range(4):
        out1.fill_(float("nan"))
        out2.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(gu.bits_of(out1), e1), i
        assert np.array_equal(gu.bits_of(out2), e2), i
        # eager work between replays
        skg.skinny_gemm_bf16(A1, B1)
        torch.cuda.synchronize()


def test_timed_entry_records_kernel_duration():
    """skinny_gemm_bf16_timed gives the same bits as skinny_gemm_bf16 and its
    events bracket the kernel itself (positive, and no longer than a pair of
    stream events recorded around the same call)."""
    torch = gu.torch_cuda()
    A, B = _problem(16, 14336, 7168)
    ref = gu.bits_of(skg.skinny_gemm_bf16(A, B, out_dtype=torch.bfloat16))
    e0, e1 = skg.HipEvent(), skg.HipEvent()
    s0 = torch.cuda.Event(enable_timing=True)
    s1 = torch.cuda.Event(enable_timing=True)
    durs, outer = [], []
    for _ in range(5):
        s0.record()
        out = skg.skinny_gemm_bf16_timed(A, B, e0, e1, out_dtype=torch.bfloat16)
        s1.record()
        torch.cuda.synchronize()
        assert np.array_equal(gu.bits_of(out), ref)
        durs.append(e0.elapsed_ms(e1))
        outer.append(s0.elapsed_time(s1))
    assert min(durs) > 0.0
    assert np.median(durs) <= np.median(outer) * 1.02


def test_graph_capture_lds_ring():
    """LDS-ring MFMA calls (both kinds, one with a K tail) captured in a
    graph: every replay equals the eager result."""
    torch = gu.torch_cuda()
    cases = [(16, 1536, 2048, MK(inner=skg.SKG_INNER_MFMA_RING_GA, split_k=1, row_tiles=1,
                                 waves_n=3, waves_k=1, depth=3, rb_per_wg=2)),
             (8, 1000, 333, MK(inner=skg.SKG_INNER_MFMA_RING, split_k=1, row_tiles=1,
                               waves_n=2, waves_k=2, depth=4))]
    s = torch.cuda.Stream()
    probs, eager, outs = [], [], []
    for (M, K, N, cfg) in cases:
        ld = gu.round8(K)
        A, B = gu.operands(inputs.make_a(M, K, N, lda=ld), inputs.make_b(K, N, ldb=ld), K)
        with torch.cuda.stream(s):
            eager.append(gu.bits_of(skg.skinny_gemm_bf16_with_config(A, B, cfg, stream=s)))
        probs.append((A, B, cfg))
        outs.append(torch.empty((M, N), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for (A, B, cfg), out in zip(probs, outs):
            skg.skinny_gemm_bf16_with_config(A, B, cfg, out=out, stream=s)
    for i in range(4):
        for out in outs:
            out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for out, e in zip(outs, eager):
            assert np.array_equal(gu.bits_of(out), e), i
        with torch.cuda.stream(s):
            A, B, cfg = probs[0]
            skg.skinny_gemm_bf16_with_config(A, B, cfg, stream=s)
        torch.cuda.synchronize()

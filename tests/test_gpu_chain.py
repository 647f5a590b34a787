"""A decode layer's chain of GEMMs captured in one HIP graph (GPU): the
router over fp32 weights, the qkv_a-style projection into its strided
buffer, the wide and the deep projection at M = 4, and a middle-tier call;
warm-up first (so split-K workspaces exist), then capture.  The eager result
of every member is checked against the oracle (all of it, or every row and
sampled columns at the largest shapes), and every replay, with eager work
between the replays, equals those results bit for bit, with the padding
columns of the strided buffer untouched."""
import numpy as np
import pytest

import latency_decode_gemm_amd as skg
from latency_decode_gemm_amd import inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def test_decode_chain_graph_replays_match_eager():
    torch = gu.torch_cuda()
    s = torch.cuda.Stream()
    chain = inputs.WORKLOADS_CHAIN["decode_chain"] + [
        dict(M=32, K=7168, N=2112, out="bf16", ldc=4096)]
    calls, refs = [], []
    for p in chain:
        M, K, N = p["M"], p["K"], p["N"]
        f32w = p.get("w") == "f32"
        A_bits = inputs.make_a(M, K, N)
        if f32w:
            A, W = gu.operands_f32w(A_bits, inputs.make_w_f32(K, N), K)
            with torch.cuda.stream(s):
                skg.skinny_gemm_f32w_warmup([(K, N)], [M], stream=s)
        else:
            A, W = gu.operands(A_bits, gu.cached_b(K, N), K)
            with torch.cuda.stream(s):
                skg.skinny_gemm_warmup([(K, N)], [M], stream=s)
        dt = torch.bfloat16 if p["out"] == "bf16" else torch.float32
        buf = torch.full((M, p["ldc"] or N), float("nan"), dtype=dt, device="cuda")
        calls.append((f32w, A, W, buf, N))
        refs.append((f32w, A_bits, inputs.make_w_f32(K, N) if f32w else gu.cached_b(K, N), K))
    fn = {True: skg.skinny_gemm_f32w, False: skg.skinny_gemm_bf16}
    with torch.cuda.stream(s):
        for (f32w, A, W, buf, N) in calls:
            fn[f32w](A, W, out=buf[:, :N], stream=s)
    torch.cuda.synchronize()
    eager = [gu.bits_of(buf) for (_, _, _, buf, _) in calls]
    for (f32w, A_bits, W_bits, K), (_, _, _, buf, N) in zip(refs, calls):
        C = buf[:, :N]
        if f32w:
            r = gu.assess_f32w(C, A_bits, W_bits, K)
        elif N * K > 2112 * 7168:
            r = gu.assess_sampled(C, A_bits, W_bits, K)
        else:
            r = gu.assess(C, A_bits, W_bits, K)
        assert r["ok"], (buf.shape, N, K, r)
        if buf.shape[1] > N:
            assert np.isnan(gu.to_f64(buf[:, N:])).all()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for (f32w, A, W, buf, N) in calls:
            fn[f32w](A, W, out=buf[:, :N], stream=s)
    for i in range(4):
        for (_, _, _, buf, N) in calls:
            buf[:, :N].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for j, (_, _, _, buf, N) in enumerate(calls):
            assert np.array_equal(gu.bits_of(buf), eager[j]), (i, j)
            if buf.shape[1] > N:
                assert np.isnan(gu.to_f64(buf[:, N:])).all()
        # eager work between replays, on the same stream
        with torch.cuda.stream(s):
            f32w, A, W, buf, N = calls[1]
            fn[f32w](A, W, stream=s)
        torch.cuda.synchronize()

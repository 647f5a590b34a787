"""Every M = 17..64 (the middle tier) on the six workload shapes at full size
(GPU), with the configuration dispatch picks: the tuned M values 24, 32, 48
and 64, and the untuned ones between them, which take the entry of the next
larger tuned M.  Router 7168 -> 256 / 384 and ragged K = 2880 -> 128 with
fp32 output, qkv_a-style 7168 -> 2112 as bf16 into a NaN-filled buffer with
ldc = 4096, wide 1536 -> 24576 and deep 14336 -> 7168 as bf16.  Every row
and a sample of 96 columns are compared with the oracle, which computes each
sampled output on its own."""
import functools

import numpy as np
import pytest

import latency_decode_gemm_amd as skg
from latency_decode_gemm_amd import inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

SHAPES = [  # K, N, output dtype, ldc
    (7168, 256, "f32", None),
    (7168, 384, "f32", None),
    (2880, 128, "f32", None),
    (7168, 2112, "bf16", 4096),
    (1536, 24576, "bf16", None),
    (14336, 7168, "bf16", None),
]


@functools.lru_cache(maxsize=1)
def _device_b(K, N):
    """The weights of one shape on the device (the tests run shape by shape)."""
    B_bits = gu.cached_b(K, N)
    return B_bits, gu.to_dev(B_bits)[:, :K]


@pytest.mark.parametrize("M", list(range(17, 65)))
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"K{s[0]}_N{s[1]}_{s[2]}"
                         + (f"_ldc{s[3]}" if s[3] else ""))
def test_every_mid_m_full_size(shape, M):
    torch = gu.torch_cuda()
    K, N, out, ldc = shape
    B_bits, B = _device_b(K, N)
    A_bits = inputs.make_a(M, K, N)
    A = gu.to_dev(A_bits)[:, :K]
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    buf = torch.full((M, ldc or N), float("nan"), dtype=dt, device="cuda")
    C = buf[:, :N]
    cfg = skg.skinny_gemm_dispatch(M, K, N)
    print(f"M={M} K={K} N={N} {out} ldc={ldc} cfg={cfg.as_tuple()}", flush=True)
    skg.skinny_gemm_bf16(A, B, out=C)
    torch.cuda.synchronize()
    r = gu.assess_sampled(C, A_bits, B_bits, K, seed=M)
    assert r["ok"], (M, K, N, cfg.as_tuple(), r)
    if ldc and ldc > N:
        # columns [N, ldc) of the strided output are untouched (still NaN)
        assert np.isnan(gu.to_f64(buf[:, N:])).all()

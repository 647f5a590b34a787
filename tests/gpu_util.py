"""Helpers for the GPU tests: host bf16 bit arrays <-> device tensors, and
comparison with the oracle."""
from __future__ import annotations

import functools

import numpy as np
import pytest

import oracle
from oracle import acceptance
from latency_decode_gemm_amd import inputs


def torch_cuda():
    torch = pytest.importorskip("torch")
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch


def to_dev(bits: np.ndarray):
    """uint16 bf16 patterns [R, ld] -> device bf16 tensor [R, ld]."""
    torch = torch_cuda()
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to("cuda").view(torch.bfloat16)


def bits_of(C) -> np.ndarray:
    """Device tensor -> raw bits (uint16 for bf16, uint32 for fp32)."""
    torch = torch_cuda()
    c = C.detach().contiguous().cpu()
    if c.dtype == torch.bfloat16:
        return c.view(torch.int16).numpy().view(np.uint16)
    return c.view(torch.int32).numpy().view(np.uint32)


def to_f64(C) -> np.ndarray:
    torch = torch_cuda()
    c = C.detach().contiguous().cpu()
    if c.dtype == torch.bfloat16:
        return oracle.bf16_decode(c.view(torch.int16).numpy().view(np.uint16))
    return c.numpy().astype(np.float64)


def operands(A_bits: np.ndarray, B_bits: np.ndarray, K: int):
    """Device views A[:, :K], B[:, :K] that keep the padded leading dimension."""
    A = to_dev(A_bits)
    B = to_dev(B_bits)
    return A[:, :K], B[:, :K]


def assess(C, A_bits, B_bits, K, C_ref=None) -> dict:
    torch = torch_cuda()
    if C_ref is None:
        C_ref = oracle.gemm_f64(A_bits, B_bits, K)
    an = acceptance.row_norms(oracle.bf16_decode(A_bits), K)
    bn = acceptance.row_norms(oracle.bf16_decode(B_bits), K)
    odt = "bf16" if C.dtype == torch.bfloat16 else "f32"
    return acceptance.assess(to_f64(C), C_ref, an, bn, odt)


@functools.lru_cache(maxsize=8)
def cached_b(K: int, N: int, ldb: int | None = None) -> np.ndarray:
    return inputs.make_b(K, N, ldb)


def round8(x: int) -> int:
    return (x + 7) // 8 * 8


def operands_f32w(A_bits: np.ndarray, W: np.ndarray, K: int):
    """Device views A[:, :K] (bf16) and W[:, :K] (fp32) that keep the padded
    leading dimensions."""
    torch = torch_cuda()
    A = to_dev(A_bits)
    Wd = torch.from_numpy(np.ascontiguousarray(W, dtype=np.float32)).to("cuda")
    return A[:, :K], Wd[:, :K]


def assess_f32w(C, A_bits, W, K, C_ref=None) -> dict:
    """The acceptance measures against the fp32-weight oracle (norms of the
    bf16-decoded activations and of the fp32 weights)."""
    torch = torch_cuda()
    if C_ref is None:
        C_ref = oracle.gemm_f32w(A_bits, W, K)
    an = acceptance.row_norms(oracle.bf16_decode(A_bits), K)
    wn = acceptance.row_norms(np.asarray(W, dtype=np.float64), K)
    odt = "bf16" if C.dtype == torch.bfloat16 else "f32"
    return acceptance.assess(to_f64(C), C_ref, an, wn, odt)


def assess_sampled(C, A_bits, B_bits, K, ncols=96, seed=0) -> dict:
    """The acceptance measures on every row and a sample of columns, the
    oracle computing each sampled output on its own (full-size shapes)."""
    torch = torch_cuda()
    N = C.shape[1]
    M = C.shape[0]
    rng = np.random.default_rng(seed)
    ns = np.sort(rng.choice(N, size=min(ncols, N), replace=False))
    ms = np.repeat(np.arange(M), ns.size)
    nn = np.tile(ns, M)
    ref = oracle.gemm_points(A_bits, B_bits, K, ms, nn).reshape(M, ns.size)
    an = acceptance.row_norms(oracle.bf16_decode(A_bits), K)
    bn = acceptance.row_norms(oracle.bf16_decode(B_bits[ns]), K)
    odt = "bf16" if C.dtype == torch.bfloat16 else "f32"
    return acceptance.assess(to_f64(C)[:, ns], ref, an, bn, odt)

"""Sampled check of a GEMM result against a plain float64 product.

The tuner checks every candidate configuration with it before the candidate
can enter a table. The bench runs it once after its timed loop.
The reference is PyTorch's float64 matmul on the CPU over the decoded inputs
of a few sampled columns: bf16 x bf16 (or bf16 x fp32) products are exact in
float64, so its own error is far below the bounds checked here.

The measures and bounds are those of the operation's acceptance rule:
  * e = max |C[m,n] - R[m,n]| / (|A_m| |B_n|) over the sampled columns, at
    most 2e-3 for fp32 output and 1e-2 for bf16 output (a zero denominator
    requires C[m,n] == 0);
  * the cosine of each row of C with the same row of R, at least 0.9999.
"""
from __future__ import annotations

import numpy as np

TOL = {"f32": 2e-3, "bf16": 1e-2}
MIN_COS = 0.9999


def _decode(torch, x: np.ndarray):
    """bf16 bit patterns (uint16) or fp32 values -> float64 tensor."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return torch.from_numpy(x).double()
    return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).double()


def sampled_check(torch, A_bits: np.ndarray, B_host: np.ndarray, C, K: int, out: str,
                  n_cols: int = 64, seed: int = 0) -> dict:
    """C[:, :N] (a device or host tensor, N = rows of B_host) against the
    float64 product on n_cols sampled columns and every row.  A_bits: [M, lda]
    bf16 bits; B_host: [N, ldb] bf16 bits, or fp32 weights.  Columns at and past
    K (padding) are never read.  Returns {'err', 'min_cos', 'tol', 'ok'}."""
    N = B_host.shape[0]
    ns = np.sort(np.random.default_rng(seed).choice(N, size=min(n_cols, N), replace=False))
    A = _decode(torch, A_bits)[:, :K]
    B = _decode(torch, B_host[ns])[:, :K]
    R = A @ B.T
    got = C[:, :N].detach().float().cpu().double()[:, torch.from_numpy(ns)]
    den = torch.outer(A.norm(dim=1), B.norm(dim=1))
    if not bool(torch.isfinite(got).all()):
        err = float("inf")
    else:
        zero = den == 0
        if bool((zero & (got != 0)).any()):
            err = float("inf")
        else:
            rel = (got - R).abs() / torch.where(zero, torch.ones_like(den), den)
            err = float(torch.where(zero, torch.zeros_like(rel), rel).max()) if rel.numel() else 0.0
    cos = []
    for m in range(got.shape[0]):
        x, y = got[m], R[m]
        nx, ny = float(x.norm()), float(y.norm())
        if nx == 0.0 and ny == 0.0:
            cos.append(1.0)
        elif nx == 0.0 or ny == 0.0 or not np.isfinite(nx):
            cos.append(0.0)
        else:
            cos.append(float(x @ y) / (nx * ny))
    min_cos = min(cos) if cos else 1.0
    tol = TOL[out]
    return {"err": err, "min_cos": min_cos, "tol": tol, "ok": err <= tol and min_cos >= MIN_COS}

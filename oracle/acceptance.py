"""Acceptance measures for comparing a GEMM result with the oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Two measures, both computed in binary64 over bf16-decoded inputs:

* normalised error  e = max_{m,n} |C[m,n] - C_ref[m,n]| / (||A_m||_2 ||B_n||_2)
  where A_m is row m of A[:, :K] and B_n row n of B[:, :K].  When the
  denominator is 0 the exact result is 0, and the entry passes only if
  C[m,n] is (+-)0.
* per-row cosine     cos(C[m,:], C_ref[m,:]); two all-zero rows count as 1,
  exactly one all-zero row as 0.

Tolerances: e <= 2e-3 for fp32 output, e <= 1e-2 for bf16 output, and every
row cosine >= 0.9999.  Sequential fp32 accumulation of bf16 products has a
normalised error of at most K * 2^-24 (about 8.5e-4 at K = 14336), and
rounding the result to bf16 adds at most 2^-9 relative, so both bounds hold
for any fp32-accumulating kernel while a bf16-accumulating one fails them.
"""
from __future__ import annotations

import numpy as np

TOL_F32 = 2e-3
TOL_BF16 = 1e-2
MIN_COS = 0.9999


def row_norms(X_dec: np.ndarray, K: int) -> np.ndarray:
    X = np.asarray(X_dec, dtype=np.float64)[:, :K]
    return np.sqrt(np.sum(X * X, axis=1))


def normalized_error(C, C_ref, a_norms, b_norms) -> float:
    C = np.asarray(C, dtype=np.float64)
    R = np.asarray(C_ref, dtype=np.float64)
    if C.shape != R.shape:
        raise ValueError(f"shape mismatch {C.shape} vs {R.shape}")
    if C.size == 0:
        return 0.0
    den = np.outer(np.asarray(a_norms, np.float64), np.asarray(b_norms, np.float64))
    diff = np.abs(C - R)
    if not np.all(np.isfinite(C)):
        return float("inf")
    zero = den == 0.0
    if np.any(zero & (C != 0.0)):
        return float("inf")
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(zero, 0.0, diff / np.where(zero, 1.0, den))
    return float(rel.max())


def row_cosines(C, C_ref) -> np.ndarray:
    C = np.asarray(C, dtype=np.float64)
    R = np.asarray(C_ref, dtype=np.float64)
    out = np.empty(C.shape[0], dtype=np.float64)
    for m in range(C.shape[0]):
        x, y = C[m], R[m]
        nx, ny = np.linalg.norm(x), np.linalg.norm(y)
        if nx == 0.0 and ny == 0.0:
            out[m] = 1.0
        elif nx == 0.0 or ny == 0.0 or not np.isfinite(nx):
            out[m] = 0.0
        else:
            out[m] = float(np.dot(x, y) / (nx * ny))
    return out


def tolerance(out_dtype: str) -> float:
    if out_dtype in ("f32", "fp32", "float32"):
        return TOL_F32
    if out_dtype in ("bf16", "bfloat16"):
        return TOL_BF16
    raise ValueError(out_dtype)


def assess(C, C_ref, a_norms, b_norms, out_dtype: str) -> dict:
    """Returns {'err', 'min_cos', 'tol', 'ok'} for one result."""
    err = normalized_error(C, C_ref, a_norms, b_norms)
    cos = row_cosines(C, C_ref) if np.asarray(C).size else np.ones(0)
    min_cos = float(cos.min()) if cos.size else 1.0
    tol = tolerance(out_dtype)
    return {"err": err, "min_cos": min_cos, "tol": tol,
            "ok": bool(err <= tol and min_cos >= MIN_COS)}

"""CPU oracle for the small-M bf16 skinny GEMM -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never imports, links
or loads it, and it imports nothing from the HIP library: the only thing the
two sides share is the seeded input generator, which the callers run and whose
output (bf16 bit patterns) they pass in here.

What it computes is the plain definition of the operation the pages describe
(PR #42562 page, "Add generic cuteDSL LL BF16 router (GEMM)", section
实现拆解 items 1-2 and the _ll_bf16_dotprod.py excerpt; PR #48597 page,
"GLM-5.2 Blackwell decode optimizations", section 实现拆解 item 3)::

    C[m, n] = sum_k dec(A[m, k]) * dec(B[n, k])      (C = A . B^T)

evaluated in binary64 with k ascending.  The fp32-weight router GEMM
(:func:`gemm_f32w`, :func:`gemm_f32w_points`, :func:`gemm_f32w_py`) is the
same sum with binary32 weights ``W[n, k]`` in place of ``dec(B[n, k])``: the
PR #48597 page lists an FP32 router GEMM and the preservation of FP32 router
weights among its parts (section 关联脉络) without printing their code, and
the reading taken here is the plain product ``C = A . W^T``.  Two
implementations of each:

* :func:`gemm_f64` / :func:`gemm_points` -- the plain C loop in ``oracle.c``
  (OpenMP over independent columns only), for every size;
* :func:`gemm_py` -- the same loop in pure Python, for tiny cases.

Both are pinned by ``tests/test_oracle_pins.py`` against one-hot and
identity inputs, closed forms, exact rational brute force and numpy's
binary64 matmul.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib: Optional[ctypes.CDLL] = None


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc -O2 -fopenmp."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
               "-fno-fast-math", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        build(force=False)
        lib = ctypes.CDLL(_LIB)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        f64p = ctypes.POINTER(ctypes.c_double)
        i32p = ctypes.POINTER(ctypes.c_int)
        lib.oracle_gemm_f64.argtypes = [u16p, u16p, f64p, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_int64, ctypes.c_int]
        lib.oracle_gemm_f64.restype = ctypes.c_int
        lib.oracle_gemm_f64_points.argtypes = [u16p, u16p, ctypes.c_int, ctypes.c_int64,
                                               ctypes.c_int64, i32p, i32p, ctypes.c_int,
                                               f64p, ctypes.c_int]
        lib.oracle_gemm_f64_points.restype = ctypes.c_int
        f32p = ctypes.POINTER(ctypes.c_float)
        lib.oracle_gemm_f32w_f64.argtypes = [u16p, f32p, f64p, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                             ctypes.c_int64, ctypes.c_int]
        lib.oracle_gemm_f32w_f64.restype = ctypes.c_int
        lib.oracle_gemm_f32w_f64_points.argtypes = [u16p, f32p, ctypes.c_int, ctypes.c_int64,
                                                    ctypes.c_int64, i32p, i32p, ctypes.c_int,
                                                    f64p, ctypes.c_int]
        lib.oracle_gemm_f32w_f64_points.restype = ctypes.c_int
        lib.oracle_round_bf16.argtypes = [ctypes.c_double]
        lib.oracle_round_bf16.restype = ctypes.c_uint16
        lib.oracle_bf16_decode.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_decode.restype = ctypes.c_double
        _lib = lib
    return _lib


def _as_u16_2d(x: np.ndarray, name: str) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype != np.uint16 or x.ndim != 2:
        raise TypeError(f"{name} must be a 2-D uint16 array of bf16 bit patterns")
    return np.ascontiguousarray(x)


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)))


def gemm_f64(A_bits: np.ndarray, B_bits: np.ndarray, K: int,
             threads: Optional[int] = None) -> np.ndarray:
    """C[M, N] in binary64 from row-major bf16 bit patterns.

    ``A_bits`` is [M, lda] and ``B_bits`` is [N, ldb] (uint16); only the first
    ``K`` columns of each row enter the sum, so padded leading dimensions work.
    """
    A = _as_u16_2d(A_bits, "A_bits")
    B = _as_u16_2d(B_bits, "B_bits")
    M, lda = A.shape
    N, ldb = B.shape
    if K < 0 or K > lda or K > ldb:
        raise ValueError("K must satisfy 0 <= K <= lda, ldb")
    C = np.zeros((M, N), dtype=np.float64)
    if M == 0 or N == 0:
        return C
    lib = _load()
    u16p = ctypes.POINTER(ctypes.c_uint16)
    rc = lib.oracle_gemm_f64(A.ctypes.data_as(u16p), B.ctypes.data_as(u16p),
                             C.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                             M, N, K, lda, ldb, N, threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_gemm_f64 rejected its arguments")
    return C


def gemm_points(A_bits: np.ndarray, B_bits: np.ndarray, K: int, ms, ns,
                threads: Optional[int] = None) -> np.ndarray:
    """C[ms[i], ns[i]] in binary64, one output at a time (sampled checks)."""
    A = _as_u16_2d(A_bits, "A_bits")
    B = _as_u16_2d(B_bits, "B_bits")
    ms = np.ascontiguousarray(ms, dtype=np.int32)
    ns = np.ascontiguousarray(ns, dtype=np.int32)
    if ms.shape != ns.shape or ms.ndim != 1:
        raise ValueError("ms and ns must be 1-D and of equal length")
    if ms.size and (ms.min() < 0 or ms.max() >= A.shape[0] or ns.min() < 0
                    or ns.max() >= B.shape[0]):
        raise ValueError("sample index out of range")
    if K < 0 or K > A.shape[1] or K > B.shape[1]:
        raise ValueError("K must satisfy 0 <= K <= lda, ldb")
    out = np.zeros(ms.size, dtype=np.float64)
    if ms.size == 0:
        return out
    lib = _load()
    u16p = ctypes.POINTER(ctypes.c_uint16)
    i32p = ctypes.POINTER(ctypes.c_int)
    rc = lib.oracle_gemm_f64_points(A.ctypes.data_as(u16p), B.ctypes.data_as(u16p), K,
                                    A.shape[1], B.shape[1], ms.ctypes.data_as(i32p),
                                    ns.ctypes.data_as(i32p), ms.size,
                                    out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                    threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_gemm_f64_points rejected its arguments")
    return out


def _as_f32_2d(x: np.ndarray, name: str) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype != np.float32 or x.ndim != 2:
        raise TypeError(f"{name} must be a 2-D float32 array")
    return np.ascontiguousarray(x)


def gemm_f32w(A_bits: np.ndarray, W: np.ndarray, K: int,
              threads: Optional[int] = None) -> np.ndarray:
    """C[M, N] in binary64 from bf16 activations ``A_bits`` [M, lda] (uint16)
    and binary32 weights ``W`` [N, ldw] (float32); the first ``K`` columns."""
    A = _as_u16_2d(A_bits, "A_bits")
    Wc = _as_f32_2d(W, "W")
    M, lda = A.shape
    N, ldw = Wc.shape
    if K < 0 or K > lda or K > ldw:
        raise ValueError("K must satisfy 0 <= K <= lda, ldw")
    C = np.zeros((M, N), dtype=np.float64)
    if M == 0 or N == 0:
        return C
    lib = _load()
    rc = lib.oracle_gemm_f32w_f64(A.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)),
                                  Wc.ctypes.data_as(ctypes.POINTER(ctypes.c_float)),
                                  C.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                  M, N, K, lda, ldw, N, threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_gemm_f32w_f64 rejected its arguments")
    return C


def gemm_f32w_points(A_bits: np.ndarray, W: np.ndarray, K: int, ms, ns,
                     threads: Optional[int] = None) -> np.ndarray:
    """C[ms[i], ns[i]] of :func:`gemm_f32w`, one output at a time."""
    A = _as_u16_2d(A_bits, "A_bits")
    Wc = _as_f32_2d(W, "W")
    ms = np.ascontiguousarray(ms, dtype=np.int32)
    ns = np.ascontiguousarray(ns, dtype=np.int32)
    if ms.shape != ns.shape or ms.ndim != 1:
        raise ValueError("ms and ns must be 1-D and of equal length")
    if ms.size and (ms.min() < 0 or ms.max() >= A.shape[0] or ns.min() < 0
                    or ns.max() >= Wc.shape[0]):
        raise ValueError("sample index out of range")
    if K < 0 or K > A.shape[1] or K > Wc.shape[1]:
        raise ValueError("K must satisfy 0 <= K <= lda, ldw")
    out = np.zeros(ms.size, dtype=np.float64)
    if ms.size == 0:
        return out
    lib = _load()
    i32p = ctypes.POINTER(ctypes.c_int)
    rc = lib.oracle_gemm_f32w_f64_points(A.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)),
                                         Wc.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), K,
                                         A.shape[1], Wc.shape[1], ms.ctypes.data_as(i32p),
                                         ns.ctypes.data_as(i32p), ms.size,
                                         out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                         threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_gemm_f32w_f64_points rejected its arguments")
    return out


def bf16_decode(bits) -> np.ndarray:
    """bf16 bit patterns -> binary64 values (exact): the 16 bits are the upper
    half of a binary32 word."""
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def round_bf16(x: float) -> int:
    """Nearest bf16 (ties to even) of a binary64 value, as a 16-bit pattern."""
    return int(_load().oracle_round_bf16(float(x)))


def _dec_py(h: int) -> float:
    """Pure-Python bf16 decode: sign, 8-bit exponent (bias 127), 7-bit
    fraction, with binary32's subnormal and special encodings."""
    s = -1.0 if (h >> 15) & 1 else 1.0
    e = (h >> 7) & 0xFF
    f = h & 0x7F
    if e == 0xFF:
        return s * float("inf") if f == 0 else float("nan")
    if e == 0:
        return s * (f / 128.0) * 2.0 ** -126
    return s * (1.0 + f / 128.0) * 2.0 ** (e - 127)


def gemm_py(A_bits, B_bits, K: int) -> list:
    """Pure-Python loop oracle for tiny cases: list of M rows of N floats."""
    A = [[int(v) for v in row] for row in np.asarray(A_bits, dtype=np.uint16)]
    B = [[int(v) for v in row] for row in np.asarray(B_bits, dtype=np.uint16)]
    C = []
    for a_row in A:
        c_row = []
        for b_row in B:
            s = 0.0
            for k in range(K):
                s += _dec_py(a_row[k]) * _dec_py(b_row[k])
            c_row.append(s)
        C.append(c_row)
    return C


def _f32_py(x) -> float:
    """A numpy binary32 value as a Python float (exact widening)."""
    return float(x)


def gemm_f32w_py(A_bits, W, K: int) -> list:
    """Pure-Python loop of :func:`gemm_f32w` for tiny cases."""
    A = [[int(v) for v in row] for row in np.asarray(A_bits, dtype=np.uint16)]
    Wr = [[_f32_py(v) for v in row] for row in np.asarray(W, dtype=np.float32)]
    C = []
    for a_row in A:
        c_row = []
        for w_row in Wr:
            s = 0.0
            for k in range(K):
                s += _dec_py(a_row[k]) * w_row[k]
            c_row.append(s)
        C.append(c_row)
    return C

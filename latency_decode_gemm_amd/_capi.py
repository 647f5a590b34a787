"""ctypes declarations for libskinny_gemm.so (see include/skinny_gemm.h).

Loading is lazy and loud: the first call that needs the library raises
``RuntimeError`` if ``libskinny_gemm.so`` has not been built.  There is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libskinny_gemm.so")

SKG_OK = 0
SKG_ERR_INVALID_ARG = 1
SKG_ERR_UNSUPPORTED = 2
SKG_ERR_MISALIGNED = 3
SKG_ERR_NOT_WARMED = 4
SKG_ERR_HIP = 5
SKG_ERR_NO_DEVICE = 6
SKG_ERR_SCRATCH_TOO_SMALL = 7

SKG_OUT_F32 = 0
SKG_OUT_BF16 = 1

SKG_BACKEND_DOT = 0
SKG_BACKEND_SPLITK = 1
SKG_BACKEND_SPLITK_2PASS = 2
SKG_BACKEND_EVEN = 3
SKG_INNER_VALU = 0
SKG_INNER_MFMA = 1
SKG_INNER_MFMA_GA = 2
SKG_INNER_VALU_GA = 3
SKG_INNER_MFMA_RING = 4
SKG_INNER_MFMA_RING_GA = 5
SKG_INNER_MFMA_RING_SYNC = 6
SKG_INNER_MFMA_RING_SHARED = 7
SKG_MAX_M = 64
SKG_MAX_M_VALU = 16
SKG_SCRATCH_SLOT_BYTES = 1 << 20
SKG_SCRATCH_PARTIAL_BYTES = 1 << 20

# Compiled (row_tiles, depth) pairs per inner product (the library's tables).
VALU_VARIANTS = ((1, 4), (1, 8), (1, 12), (2, 2), (2, 4), (2, 8), (4, 2), (4, 4))
MFMA_VARIANTS = ((1, 2), (1, 3), (1, 4), (1, 6), (2, 1), (2, 2), (2, 3), (2, 4), (4, 1),
                 (4, 2))
# the barrier kinds (M <= 16): SKG_INNER_MFMA_RING_SYNC, and the shared
# activation ring SKG_INNER_MFMA_RING_SHARED (depth >= 3)
SYNC_VARIANTS = ((1, 2), (1, 3), (1, 4), (1, 6), (2, 1), (2, 2), (2, 3), (2, 4))
SHARED_VARIANTS = tuple(v for v in SYNC_VARIANTS if v[1] >= 3)

# Every function the header declares, with (restype, argtypes).
_i = ctypes.c_int
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_ip = ctypes.POINTER(ctypes.c_int)


class SkgConfig(ctypes.Structure):
    """Mirror of ``skg_config``."""
    _fields_ = [("backend", ctypes.c_int32), ("inner", ctypes.c_int32),
                ("split_k", ctypes.c_int32), ("row_tiles", ctypes.c_int32),
                ("waves_n", ctypes.c_int32), ("waves_k", ctypes.c_int32),
                ("depth", ctypes.c_int32), ("rb_per_wg", ctypes.c_int32)]

    FIELDS = ("backend", "inner", "split_k", "row_tiles", "waves_n", "waves_k", "depth",
              "rb_per_wg")

    def as_tuple(self):
        return tuple(getattr(self, f) for f in self.FIELDS)

    def as_dict(self):
        return {f: getattr(self, f) for f in self.FIELDS}

    @classmethod
    def make(cls, backend=None, inner=SKG_INNER_VALU, split_k=1, row_tiles=1, waves_n=1,
             waves_k=1, depth=4, rb_per_wg=1):
        if backend is None:
            backend = SKG_BACKEND_DOT if split_k == 1 else SKG_BACKEND_SPLITK
        return cls(backend, inner, split_k, row_tiles, waves_n, waves_k, depth, rb_per_wg)

    def __eq__(self, other):
        return isinstance(other, SkgConfig) and self.as_tuple() == other.as_tuple()

    def __hash__(self):
        return hash(self.as_tuple())

    def __repr__(self):
        return "SkgConfig(" + ", ".join(f"{k}={v}" for k, v in self.as_dict().items()) + ")"


_cfgp = ctypes.POINTER(SkgConfig)

SIGNATURES = {
    "skinny_gemm_bf16": (_i, [_vp, _vp, _vp, _i, _i, _i, _i64, _i64, _i64, _i, _vp]),
    "skinny_gemm_bf16_noalloc": (_i, [_vp, _vp, _vp, _i, _i, _i, _i64, _i64, _i64, _i, _vp]),
    "skinny_gemm_bf16_timed": (_i, [_vp, _vp, _vp, _i, _i, _i, _i64, _i64, _i64, _i, _vp,
                                    _vp, _vp]),
    "skinny_gemm_bf16_with_config": (_i, [_vp, _vp, _vp, _i, _i, _i, _i64, _i64, _i64, _i,
                                          _vp, _cfgp]),
    "skinny_gemm_dispatch": (_i, [_i, _i, _i, _cfgp]),
    "skinny_gemm_check_config": (_i, [_i, _i, _i, _cfgp]),
    "skinny_gemm_workspace_bytes": (_i, [_i, _i, _i, _cfgp, ctypes.POINTER(ctypes.c_size_t)]),
    "skinny_gemm_warmup_keys": (_i, [_ip, _i, _ip, _i, _cfgp, _i, _ip]),
    "skinny_gemm_warmup": (_i, [_ip, _i, _ip, _i, _vp, _ip]),
    "skinny_gemm_f32w": (_i, [_vp, _vp, _vp, _i, _i, _i, _i64, _i64, _i64, _i, _vp]),
    "skinny_gemm_f32w_timed": (_i, [_vp, _vp, _vp, _i, _i, _i, _i64, _i64, _i64, _i, _vp,
                                    _vp, _vp]),
    "skinny_gemm_f32w_with_config": (_i, [_vp, _vp, _vp, _i, _i, _i, _i64, _i64, _i64, _i,
                                          _vp, _cfgp]),
    "skinny_gemm_f32w_dispatch": (_i, [_i, _i, _i, _cfgp]),
    "skinny_gemm_f32w_check_config": (_i, [_i, _i, _i, _cfgp]),
    "skinny_gemm_f32w_warmup_keys": (_i, [_ip, _i, _ip, _i, _cfgp, _i, _ip]),
    "skinny_gemm_f32w_warmup": (_i, [_ip, _i, _ip, _i, _vp, _ip]),
    "skinny_gemm_max_m": (_i, [_i, _i, _ip]),
    "skinny_gemm_last_hip_error": (_i, []),
    "skinny_gemm_available": (_i, []),
    "skinny_gemm_stream_read": (_i, [_vp, ctypes.c_size_t, _vp, _vp]),
    "skinny_gemm_strerror": (ctypes.c_char_p, [_i]),
}

_lib = None
_lock = threading.Lock()


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError(
                        f"{LIB_PATH} is missing: build it with "
                        "`python -m latency_decode_gemm_amd.build` (there is no fallback)")
                # The library needs the HIP runtime that torch, whose device
                # memory and streams it is handed, already uses: with torch
                # loaded first, the library's libamdhip64.so.7 dependency
                # resolves to torch's copy; loaded before it, the library
                # would bind the system runtime and the process would hold
                # two runtimes that do not share streams or loaded kernels.
                try:
                    import torch  # noqa: F401
                except ImportError:
                    pass
                dll = ctypes.CDLL(LIB_PATH)
                for name, (res, args) in SIGNATURES.items():
                    fn = getattr(dll, name)
                    fn.restype = res
                    fn.argtypes = args
                _lib = dll
    return _lib


class HipEvent:
    """A timing hipEvent_t (for skinny_gemm_bf16_timed), via the HIP runtime."""
    _hip = None

    @classmethod
    def _rt(cls):
        if cls._hip is None:
            hip = ctypes.CDLL("libamdhip64.so")
            hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
            cls._hip = hip
        return cls._hip

    def __init__(self):
        self.handle = ctypes.c_void_p()
        if self._rt().hipEventCreate(ctypes.byref(self.handle)) != 0:
            raise RuntimeError("hipEventCreate failed")

    def elapsed_ms(self, end: "HipEvent") -> float:
        ms = ctypes.c_float()
        if self._rt().hipEventSynchronize(end.handle) != 0:
            raise RuntimeError("hipEventSynchronize failed")
        if self._rt().hipEventElapsedTime(ctypes.byref(ms), self.handle, end.handle) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def __del__(self):
        if self._hip is not None and self.handle:
            self._hip.hipEventDestroy(self.handle)


class SkinnyGemmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib().skinny_gemm_strerror(status).decode()
        if status == SKG_ERR_HIP:
            msg += f", hipError_t {lib().skinny_gemm_last_hip_error()}"
        super().__init__(f"{where}: status {status} ({msg})")


def check(status: int, where: str) -> None:
    if status != SKG_OK:
        raise SkinnyGemmError(status, where)

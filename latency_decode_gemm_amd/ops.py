"""Python entry points with the C ABI's names (argument marshalling only).

Tensors are PyTorch device tensors; every computation runs in the HIP
library.  dtype guards live here because the C ABI takes ``void*``: both
operands must be bf16 (the router gate on the PR #42562 page, section
评论区精华, requires bf16 for the activations and for the weight), except
for the ``skinny_gemm_f32w*`` entry points, whose weights are fp32.
"""
from __future__ import annotations

import ctypes
from typing import Iterable, Optional, Sequence, Tuple

from . import _capi
from ._capi import SkgConfig, check


def _torch():
    import torch
    return torch


def _stream_handle(stream, device):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _round8(x: int) -> int:
    return (x + 7) // 8 * 8


def _marshal(A, B, out, out_dtype, f32w=False):
    torch = _torch()
    if f32w:
        if A.dtype != torch.bfloat16 or B.dtype != torch.float32:
            raise TypeError(f"A must be torch.bfloat16 and W torch.float32 (got {A.dtype}, "
                            f"{B.dtype})")
    elif A.dtype != torch.bfloat16 or B.dtype != torch.bfloat16:
        raise TypeError(f"A and B must be torch.bfloat16 (got {A.dtype}, {B.dtype})")
    if A.dim() != 2 or B.dim() != 2:
        raise ValueError("A must be [M, K] and B [N, K]")
    M, K = A.shape
    N, Kb = B.shape
    if Kb != K:
        raise ValueError(f"inner dimensions differ: A is [{M}, {K}], B is [{N}, {Kb}]")
    if not (A.is_cuda and B.is_cuda):
        raise ValueError("A and B must be device tensors")
    if (K > 1 and A.stride(1) != 1 and M > 0) or (K > 1 and B.stride(1) != 1 and N > 0):
        raise ValueError("rows of A and B must be contiguous (stride 1 along K)")
    if out is None:
        dt = torch.float32 if out_dtype is None else out_dtype
        out = torch.empty((M, N), dtype=dt, device=A.device)
    if out.dim() != 2 or tuple(out.shape) != (M, N):
        raise ValueError(f"out must be [{M}, {N}]")
    if out.dtype == torch.float32:
        odt = _capi.SKG_OUT_F32
    elif out.dtype == torch.bfloat16:
        odt = _capi.SKG_OUT_BF16
    else:
        raise TypeError(f"out must be float32 or bfloat16 (got {out.dtype})")
    if N > 1 and out.stride(1) != 1:
        raise ValueError("rows of out must be contiguous")
    if out.device != A.device or B.device != A.device:
        raise ValueError("A, B and out must be on the same device")
    # a stride is only meaningful when there is a second row
    lda = A.stride(0) if M > 1 else max(_round8(K), 8)
    ldb = B.stride(0) if N > 1 else max(_round8(K), 8)  # elements of B's dtype
    ldc = out.stride(0) if M > 1 else max(N, 1)
    return M, N, K, lda, ldb, ldc, odt, out


def skinny_gemm_bf16(A, B, out=None, out_dtype=None, stream=None):
    """C = A . B^T (A [M, K], B [N, K], bf16; M <= 64) into ``out`` (fp32 or
    bf16, may be a strided view).  Returns ``out``."""
    M, N, K, lda, ldb, ldc, odt, out = _marshal(A, B, out, out_dtype)
    st = _capi.lib().skinny_gemm_bf16(A.data_ptr(), B.data_ptr(), out.data_ptr(), M, N, K,
                                      lda, ldb, ldc, odt, _stream_handle(stream, A.device))
    check(st, "skinny_gemm_bf16")
    return out


def skinny_gemm_bf16_noalloc(A, B, out, stream=None):
    """As :func:`skinny_gemm_bf16`, allocating nothing: ``out`` must be given,
    and the split-K workspace is the library's static per-GPU scratch (calls
    that overlap on one GPU race on it).  Raises SkinnyGemmError with
    SKG_ERR_SCRATCH_TOO_SMALL when the shape's workspace does not fit."""
    if out is None:
        raise ValueError("skinny_gemm_bf16_noalloc needs `out` (it allocates nothing)")
    M, N, K, lda, ldb, ldc, odt, out = _marshal(A, B, out, None)
    st = _capi.lib().skinny_gemm_bf16_noalloc(A.data_ptr(), B.data_ptr(), out.data_ptr(), M, N,
                                              K, lda, ldb, ldc, odt,
                                              _stream_handle(stream, A.device))
    check(st, "skinny_gemm_bf16_noalloc")
    return out


def skinny_gemm_bf16_timed(A, B, start_event, stop_event, out=None, out_dtype=None, stream=None):
    """As :func:`skinny_gemm_bf16`; the kernel's own start and end are
    recorded in ``start_event`` / ``stop_event`` (:class:`HipEvent` or raw
    hipEvent_t handles)."""
    M, N, K, lda, ldb, ldc, odt, out = _marshal(A, B, out, out_dtype)
    h0 = getattr(start_event, "handle", start_event)
    h1 = getattr(stop_event, "handle", stop_event)
    st = _capi.lib().skinny_gemm_bf16_timed(A.data_ptr(), B.data_ptr(), out.data_ptr(), M, N, K,
                                            lda, ldb, ldc, odt, _stream_handle(stream, A.device),
                                            h0, h1)
    check(st, "skinny_gemm_bf16_timed")
    return out


def skinny_gemm_bf16_with_config(A, B, cfg: SkgConfig, out=None, out_dtype=None, stream=None):
    """As :func:`skinny_gemm_bf16` with an explicit kernel configuration."""
    M, N, K, lda, ldb, ldc, odt, out = _marshal(A, B, out, out_dtype)
    st = _capi.lib().skinny_gemm_bf16_with_config(
        A.data_ptr(), B.data_ptr(), out.data_ptr(), M, N, K, lda, ldb, ldc, odt,
        _stream_handle(stream, A.device), ctypes.byref(cfg))
    check(st, "skinny_gemm_bf16_with_config")
    return out


def skinny_gemm_dispatch(M: int, K: int, N: int) -> SkgConfig:
    cfg = SkgConfig()
    check(_capi.lib().skinny_gemm_dispatch(M, K, N, ctypes.byref(cfg)), "skinny_gemm_dispatch")
    return cfg


def skinny_gemm_check_config(M: int, K: int, N: int, cfg: SkgConfig) -> bool:
    return _capi.lib().skinny_gemm_check_config(M, K, N, ctypes.byref(cfg)) == _capi.SKG_OK


def skinny_gemm_workspace_bytes(M: int, K: int, N: int, cfg: SkgConfig) -> int:
    n = ctypes.c_size_t(0)
    check(_capi.lib().skinny_gemm_workspace_bytes(M, K, N, ctypes.byref(cfg), ctypes.byref(n)),
          "skinny_gemm_workspace_bytes")
    return int(n.value)


def skinny_gemm_f32w(A, W, out=None, out_dtype=None, stream=None):
    """C = A . W^T with A [M, K] bf16 and fp32 weights W [N, K] (the router
    GEMM over fp32 weights; M <= 16) into ``out`` (fp32 or bf16).  Returns
    ``out``."""
    M, N, K, lda, ldw, ldc, odt, out = _marshal(A, W, out, out_dtype, f32w=True)
    st = _capi.lib().skinny_gemm_f32w(A.data_ptr(), W.data_ptr(), out.data_ptr(), M, N, K,
                                      lda, ldw, ldc, odt, _stream_handle(stream, A.device))
    check(st, "skinny_gemm_f32w")
    return out


def skinny_gemm_f32w_timed(A, W, start_event, stop_event, out=None, out_dtype=None,
                           stream=None):
    """As :func:`skinny_gemm_f32w`, recording the kernel's own start and end."""
    M, N, K, lda, ldw, ldc, odt, out = _marshal(A, W, out, out_dtype, f32w=True)
    h0 = getattr(start_event, "handle", start_event)
    h1 = getattr(stop_event, "handle", stop_event)
    st = _capi.lib().skinny_gemm_f32w_timed(A.data_ptr(), W.data_ptr(), out.data_ptr(), M, N, K,
                                            lda, ldw, ldc, odt, _stream_handle(stream, A.device),
                                            h0, h1)
    check(st, "skinny_gemm_f32w_timed")
    return out


def skinny_gemm_f32w_with_config(A, W, cfg: SkgConfig, out=None, out_dtype=None, stream=None):
    """As :func:`skinny_gemm_f32w` with an explicit kernel configuration."""
    M, N, K, lda, ldw, ldc, odt, out = _marshal(A, W, out, out_dtype, f32w=True)
    st = _capi.lib().skinny_gemm_f32w_with_config(
        A.data_ptr(), W.data_ptr(), out.data_ptr(), M, N, K, lda, ldw, ldc, odt,
        _stream_handle(stream, A.device), ctypes.byref(cfg))
    check(st, "skinny_gemm_f32w_with_config")
    return out


def skinny_gemm_f32w_dispatch(M: int, K: int, N: int) -> SkgConfig:
    cfg = SkgConfig()
    check(_capi.lib().skinny_gemm_f32w_dispatch(M, K, N, ctypes.byref(cfg)),
          "skinny_gemm_f32w_dispatch")
    return cfg


def skinny_gemm_f32w_check_config(M: int, K: int, N: int, cfg: SkgConfig) -> bool:
    return _capi.lib().skinny_gemm_f32w_check_config(M, K, N, ctypes.byref(cfg)) == _capi.SKG_OK


def _pairs(shapes: Sequence[Tuple[int, int]], m_values: Iterable[int]):
    flat = [v for kn in shapes for v in (int(kn[0]), int(kn[1]))]
    ms = [int(m) for m in m_values]
    kn_arr = (ctypes.c_int * max(len(flat), 1))(*flat)
    m_arr = (ctypes.c_int * max(len(ms), 1))(*ms)
    return kn_arr, len(flat) // 2, m_arr, len(ms)


def _warmup_keys(fn_name, shapes, m_values):
    kn_arr, ns, m_arr, nm = _pairs(shapes, m_values)
    fn = getattr(_capi.lib(), fn_name)
    n = ctypes.c_int(0)
    check(fn(kn_arr, ns, m_arr, nm, None, 0, ctypes.byref(n)), fn_name)
    buf = (SkgConfig * max(n.value, 1))()
    check(fn(kn_arr, ns, m_arr, nm, buf, n.value, ctypes.byref(n)), fn_name)
    return [SkgConfig(*buf[i].as_tuple()) for i in range(n.value)]


def _warmup(fn_name, shapes, m_values, stream, device):
    torch = _torch()
    device = torch.device("cuda", torch.cuda.current_device()) if device is None else device
    kn_arr, ns, m_arr, nm = _pairs(shapes, m_values)
    n = ctypes.c_int(0)
    with torch.cuda.device(device):
        check(getattr(_capi.lib(), fn_name)(kn_arr, ns, m_arr, nm,
                                            _stream_handle(stream, device), ctypes.byref(n)),
              fn_name)
    return int(n.value)


def skinny_gemm_warmup_keys(shapes: Sequence[Tuple[int, int]], m_values: Iterable[int]):
    """Distinct dispatch results over (K, N) in ``shapes`` x M in
    ``m_values``, first-seen order."""
    return _warmup_keys("skinny_gemm_warmup_keys", shapes, m_values)


def skinny_gemm_warmup(shapes: Sequence[Tuple[int, int]], m_values: Iterable[int],
                       stream=None, device=None) -> int:
    """Loads code, sizes the stream's split-K workspace and runs each distinct
    configuration once.  Returns the number of distinct configurations."""
    return _warmup("skinny_gemm_warmup", shapes, m_values, stream, device)


def skinny_gemm_f32w_warmup_keys(shapes: Sequence[Tuple[int, int]], m_values: Iterable[int]):
    """As :func:`skinny_gemm_warmup_keys` for fp32 weights."""
    return _warmup_keys("skinny_gemm_f32w_warmup_keys", shapes, m_values)


def skinny_gemm_f32w_warmup(shapes: Sequence[Tuple[int, int]], m_values: Iterable[int],
                            stream=None, device=None) -> int:
    """As :func:`skinny_gemm_warmup` for fp32 weights."""
    return _warmup("skinny_gemm_f32w_warmup", shapes, m_values, stream, device)


def skinny_gemm_stream_read(src, sink, nbytes: Optional[int] = None, stream=None):
    """Streams ``nbytes`` (default: all) bytes of the device tensor ``src``
    through the GEMM's load form and XOR-folds them into ``sink`` (an int32
    device tensor of >= 512 elements, one word per workgroup): the measured
    streaming-read ceiling."""
    torch = _torch()
    n = src.numel() * src.element_size() if nbytes is None else int(nbytes)
    if not (src.is_cuda and sink.is_cuda) or sink.dtype != torch.int32 or sink.numel() < 512:
        raise ValueError("src and sink must be device tensors, sink int32 with >= 512 elements")
    check(_capi.lib().skinny_gemm_stream_read(src.data_ptr(), n, sink.data_ptr(),
                                              _stream_handle(stream, src.device)),
          "skinny_gemm_stream_read")
    return sink


def skinny_gemm_max_m(K: int, N: int) -> int:
    """The measured crossover for (K, N): use this library up to this M."""
    m = ctypes.c_int(0)
    check(_capi.lib().skinny_gemm_max_m(K, N, ctypes.byref(m)), "skinny_gemm_max_m")
    return int(m.value)


def skinny_gemm_last_hip_error() -> int:
    return int(_capi.lib().skinny_gemm_last_hip_error())


def skinny_gemm_available() -> bool:
    return bool(_capi.lib().skinny_gemm_available())


def skinny_gemm_strerror(status: int) -> str:
    return _capi.lib().skinny_gemm_strerror(status).decode()

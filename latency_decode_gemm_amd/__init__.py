"""MI355X (gfx950) small-M bf16 "skinny" GEMM: C = A . B^T for M <= 16, with a
middle tier to M <= 64 and a router GEMM over fp32 weights.

The computation runs in ``libskinny_gemm.so`` (hand-written HIP kernels behind
the C ABI in ``include/skinny_gemm.h``); this package only marshals PyTorch
tensors into that ABI.  ``inputs`` holds the seeded synthetic-input recipe.
"""
from ._capi import (SKG_BACKEND_DOT, SKG_BACKEND_EVEN, SKG_BACKEND_SPLITK, SKG_BACKEND_SPLITK_2PASS, SKG_ERR_HIP, SKG_ERR_INVALID_ARG,
                    SKG_ERR_MISALIGNED, SKG_ERR_NO_DEVICE, SKG_ERR_NOT_WARMED, SKG_ERR_SCRATCH_TOO_SMALL,
                    SKG_ERR_UNSUPPORTED, SKG_INNER_MFMA, SKG_INNER_MFMA_GA,
                    SKG_INNER_MFMA_RING, SKG_INNER_MFMA_RING_GA, SKG_INNER_MFMA_RING_SHARED,
                    SKG_INNER_MFMA_RING_SYNC, SKG_INNER_VALU,
                    SKG_INNER_VALU_GA, SKG_MAX_M, SKG_MAX_M_VALU, SKG_OK,
                    SKG_OUT_BF16, SKG_OUT_F32, SKG_SCRATCH_PARTIAL_BYTES, SKG_SCRATCH_SLOT_BYTES,
                    HipEvent, SkgConfig, SkinnyGemmError)
from .ops import (skinny_gemm_available, skinny_gemm_bf16, skinny_gemm_bf16_noalloc,
                  skinny_gemm_bf16_timed,
                  skinny_gemm_bf16_with_config, skinny_gemm_f32w, skinny_gemm_f32w_check_config,
                  skinny_gemm_f32w_dispatch, skinny_gemm_f32w_timed,
                  skinny_gemm_f32w_warmup, skinny_gemm_f32w_warmup_keys,
                  skinny_gemm_f32w_with_config,
                  skinny_gemm_check_config, skinny_gemm_dispatch, skinny_gemm_last_hip_error,
                  skinny_gemm_max_m,
                  skinny_gemm_stream_read,
                  skinny_gemm_strerror,
                  skinny_gemm_warmup, skinny_gemm_warmup_keys, skinny_gemm_workspace_bytes)

__all__ = [n for n in dir() if n.startswith(("skinny_gemm", "SKG_", "Skg", "Skinny", "Hip"))]

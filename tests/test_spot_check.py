"""The sampled float64 check that the tuner and the bench use (not the
oracle) agrees with the oracle's results and rejects what the acceptance rule
rejects."""
import numpy as np
import torch

import oracle
from latency_decode_gemm_amd import inputs, spot_check

M, K, N, LD = 5, 1003, 77, 1008


def _operands():
    return inputs.make_a(M, K, N, lda=LD), inputs.make_b(K, N, ldb=LD)


def test_oracle_results_pass_for_both_output_types_and_weight_kinds():
    A, B = _operands()
    ref = oracle.gemm_f64(A, B, K)
    r = spot_check.sampled_check(torch, A, B, torch.from_numpy(ref.astype(np.float32)), K, "f32",
                                 n_cols=N)
    assert r["ok"] and r["err"] < 1e-7, r
    r = spot_check.sampled_check(torch, A, B, torch.from_numpy(ref.astype(np.float32)).bfloat16(),
                                 K, "bf16", n_cols=N)
    assert r["ok"] and r["err"] < 5e-3, r
    W = inputs.make_w_f32(K, N)
    ref = oracle.gemm_f32w(A, W, K)
    r = spot_check.sampled_check(torch, A, W, torch.from_numpy(ref.astype(np.float32)), K, "f32",
                                 n_cols=N)
    assert r["ok"] and r["err"] < 1e-7, r


def test_planted_errors_fail():
    A, B = _operands()
    ref = torch.from_numpy(oracle.gemm_f64(A, B, K).astype(np.float32))
    bad = ref.clone()
    bad[2, 5] += 1.0  # about 3e-2 of |A_2| |B_5|
    assert not spot_check.sampled_check(torch, A, B, bad, K, "f32", n_cols=N)["ok"]
    bad = ref.clone()
    bad[0, 0] = float("nan")
    assert not spot_check.sampled_check(torch, A, B, bad, K, "f32", n_cols=N)["ok"]
    # a row of A that is zero makes the exact result zero: only +-0 passes
    A0 = A.copy()
    A0[1, :K] = 0
    ref0 = torch.from_numpy(oracle.gemm_f64(A0, B, K).astype(np.float32))
    assert spot_check.sampled_check(torch, A0, B, ref0, K, "f32", n_cols=N)["ok"]
    ref0[1, 3] = 1e-30
    assert not spot_check.sampled_check(torch, A0, B, ref0, K, "f32", n_cols=N)["ok"]


def test_padding_past_k_is_not_read():
    A, B = _operands()
    ref = torch.from_numpy(oracle.gemm_f64(A, B, K).astype(np.float32))
    A2, B2 = A.copy(), B.copy()
    A2[:, K:] = 0x7FC0  # NaN in the padding columns
    B2[:, K:] = 0x7FC0
    assert spot_check.sampled_check(torch, A2, B2, ref, K, "f32", n_cols=N)["ok"]

"""Pins for oracle.gemm and oracle.linear.

Independent references: a brute-force triple loop in Python floats for the
products on dequantized operands (tiny shapes, including a partial outer
block and an NVFP4 x FP8 mix), and unbiasedness of the backward products
(TetraJet-v2 technical summary, section 2.A: the gradient estimates are
unbiased; section 2.C: the Hadamard transforms cancel).
"""
import numpy as np
import pytest

from oracle import gemm, linear, quant


@pytest.mark.parametrize("I,J,K", [(16, 16, 16), (32, 48, 256), (7, 5, 144)])
def test_gemm_vs_bruteforce(I, J, K):
    r = np.random.default_rng(I * J + K)
    a = quant.quantize(r.standard_normal((I, K)).astype(np.float32))
    b = quant.quantize((r.standard_normal((J, K)) * 0.02).astype(np.float32), rounding="sr", seed=1, offset=2)
    ref = gemm.gemm_nt_bruteforce(quant.dequantize_f64(a), quant.dequantize_f64(b))
    np.testing.assert_allclose(gemm.gemm_nt_f64(a, b), ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_gemm_mixed_fp8_vs_bruteforce():
    r = np.random.default_rng(3)
    a = quant.quantize(r.standard_normal((9, 160)).astype(np.float32), rounding="sr", seed=3, offset=0)
    b = quant.quantize(r.standard_normal((11, 160)).astype(np.float32), fmt="fp8", rounding="sr", seed=3, offset=1)
    ref = gemm.gemm_nt_bruteforce(quant.dequantize_f64(a), quant.dequantize_f64(b))
    np.testing.assert_allclose(gemm.gemm_nt_f64(a, b), ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def _inputs(M, N, K, seed):
    r = np.random.default_rng(seed)
    X = r.standard_normal((M, K)).astype(np.float32)
    W = (r.standard_normal((N, K)) * 0.02).astype(np.float32)
    dY = (r.standard_normal((M, N)) * 0.01).astype(np.float32)
    return X, W, dY


def test_forward_is_product_of_rtn_operands():
    X, W, _ = _inputs(32, 16, 64, 0)
    out = linear.linear_fwd(X, W)
    ref = gemm.gemm_nt_bruteforce(quant.dequantize_f64(out["Xq"]), quant.dequantize_f64(out["Wq"]))
    np.testing.assert_allclose(out["Y"], ref, rtol=1e-12, atol=1e-15)
    # forward error vs the unquantized product is at quantization level
    rel = np.linalg.norm(out["Y"] - X.astype(np.float64) @ W.T.astype(np.float64)) / np.linalg.norm(X @ W.T)
    assert 1e-3 < rel < 0.3


@pytest.mark.parametrize("use_plan", [False, True])
def test_backward_unbiased(use_plan):
    M, N, K = 64, 32, 64
    X, W, dY = _inputs(M, N, K, 1)
    plan = linear.Plan.from_outliers(K, [3, 17, 30, 31, 40, 41, 42, 43, 50, 51, 52, 53, 60, 61, 62, 63]) \
        if use_plan else None
    fwd = linear.linear_fwd(X, W, plan)
    if plan is None:
        Xh = quant.dequantize_f64(fwd["Xq"])
        Wh = quant.dequantize_f64(fwd["Wq"])
    else:
        Xh = np.zeros((M, K)); Wh = np.zeros((N, K))
        Xh[:, plan.rest] = quant.dequantize_f64(fwd["Xq"]); Xh[:, plan.outliers] = quant.dequantize_f64(fwd["X8"])
        Wh[:, plan.rest] = quant.dequantize_f64(fwd["Wq"]); Wh[:, plan.outliers] = quant.dequantize_f64(fwd["W8"])
    dY64 = dY.astype(np.float64)
    dX_true = dY64 @ Wh
    dW_true = dY64.T @ Xh
    errs = {}
    for S in (16, 256):
        dX = np.zeros((M, K)); dW = np.zeros((N, K))
        for s in range(S):
            b = linear.linear_bwd(dY, fwd, seed=1234, offset=8 * s, plan=plan)
            dX += b["dX"]; dW += b["dW"]
        errs[S] = (np.linalg.norm(dX / S - dX_true) / np.linalg.norm(dX_true),
                   np.linalg.norm(dW / S - dW_true) / np.linalg.norm(dW_true))
    for i in range(2):
        # error of the mean shrinks like 1/sqrt(S): 16x more samples -> ~4x smaller
        assert errs[256][i] < errs[16][i] / 2.5
        assert errs[256][i] < 0.05


def test_backward_without_rht_and_quantization_noise_level():
    X, W, dY = _inputs(64, 32, 64, 2)
    fwd = linear.linear_fwd(X, W)
    b = linear.linear_bwd(dY, fwd, seed=0, offset=0, rht=False)
    assert b["mask_dx"] is None
    Wh = quant.dequantize_f64(fwd["Wq"])
    ref = dY.astype(np.float64) @ Wh
    rel = np.linalg.norm(b["dX"] - ref) / np.linalg.norm(ref)
    assert 1e-3 < rel < 0.5

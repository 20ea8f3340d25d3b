"""Forward and backward of the NVFP4 linear layer (oracle; test infrastructure only).

Y = X W^T with X [M, K] (tokens x in-features) and W [N, K].

Forward (TetraJet-v2 technical summary, section 2.A): X and W are quantized
with round-to-nearest in 1x16 groups along K; Y is their product.

Backward (section 2.A "unbiased gradient estimation" and section 2.C RHT).
Reading taken for "estimate X-hat instead of X": the backward pass re-uses the
forward's *dequantized* tensors X-hat and W-hat, so both gradients are unbiased
estimates of the gradients of the quantized forward.  Each backward operand
is the 16-wide random Hadamard transform along the reduction dimension
followed by stochastic rounding, with one Philox offset per operand:

  dX = Q(dY T_N) . Q(T_N^T W-hat)     dY grouped along N        offset + 0
                                       W-hat re-grouped along N  offset + 1
  dW = Q(dY^T T_M) . Q(T_M^T X-hat)   dY re-grouped along M     offset + 2
                                       X-hat re-grouped along M  offset + 3

Both operands of one product share one sign mask (rht_signs(seed, offset+0)
for dX, rht_signs(seed, offset+2) for dW), so the transforms cancel in the
exact product.

FP6 x FP4 (the mixed-precision strategy the pages name as future work,
section 5; reading: the gradient operand gets the wider element): with
grad_fmt="nvfp6" the two dY operands are double-block NVFP6 (E2M3 elements,
same scales, offsets, masks and SR rule) while W-hat and X-hat stay NVFP4.

OutControl (section 2.C): a static, sorted list O of input channels (the top
p% from calibration) stays in FP8 in forward and backward; the remaining
channels O-bar (sorted) are compacted and quantized to NVFP4 over the
compacted order.  dY is not indexed by input channels and stays NVFP4.

  Y        = X_Obar W_Obar^T (NVFP4)          + X_O W_O^T (FP8, RNE)
  dX[:, Obar] = Q(dY T_N) . Q(T_N^T W-hat_Obar) (NVFP4)
  dX[:, O]    = Q(dY T_N) . Q8(T_N^T W-hat_O)    (FP8, SR, offset + 4)
  dW[:, Obar] = Q(dY^T T_M) . Q(T_M^T X-hat_Obar)
  dW[:, O]    = Q(dY^T T_M) . Q8(T_M^T X-hat_O)   (FP8, SR, offset + 5)
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import philox
from .gemm import gemm_nt_f64
from .quant import QTensor, dequantize, quantize


@dataclass
class Plan:
    outliers: np.ndarray  # sorted channel indices kept in FP8
    rest: np.ndarray  # sorted complement (NVFP4)

    @staticmethod
    def from_outliers(K: int, outliers) -> "Plan":
        o = np.sort(np.asarray(outliers, dtype=np.int64))
        mask = np.ones(K, dtype=bool)
        mask[o] = False
        return Plan(o, np.nonzero(mask)[0].astype(np.int64))


def linear_fwd(X: np.ndarray, W: np.ndarray, plan: Plan | None = None) -> dict:
    """X fp32 [M, K] (values of the bf16 input), W fp32 [N, K] masters."""
    X = np.asarray(X, dtype=np.float32)
    W = np.asarray(W, dtype=np.float32)
    if plan is None:
        Xq = quantize(X, grouping="row", fmt="nvfp4", rounding="rtn")
        Wq = quantize(W, grouping="row", fmt="nvfp4", rounding="rtn")
        return {"Xq": Xq, "Wq": Wq, "Y": gemm_nt_f64(Xq, Wq)}
    Xq = quantize(X[:, plan.rest], grouping="row", fmt="nvfp4", rounding="rtn")
    Wq = quantize(W[:, plan.rest], grouping="row", fmt="nvfp4", rounding="rtn")
    X8 = quantize(X[:, plan.outliers], grouping="row", fmt="fp8", rounding="rtn")
    W8 = quantize(W[:, plan.outliers], grouping="row", fmt="fp8", rounding="rtn")
    Y = gemm_nt_f64(Xq, Wq) + gemm_nt_f64(X8, W8)
    return {"Xq": Xq, "Wq": Wq, "X8": X8, "W8": W8, "Y": Y}


def linear_bwd(dY: np.ndarray, saved: dict, seed: int, offset: int, rht: bool = True,
               plan: Plan | None = None, grad_fmt: str = "nvfp4") -> dict:
    """dY fp32 [M, N] (values of the bf16 gradient); saved = linear_fwd's result; grad_fmt "nvfp4"
    or "nvfp6" (the format of the two dY operands)."""
    dY = np.asarray(dY, dtype=np.float32)
    Xq: QTensor = saved["Xq"]
    Wq: QTensor = saved["Wq"]
    M, N = dY.shape
    mask_dx = philox.rht_signs(seed, offset + 0) if rht else None
    mask_dw = philox.rht_signs(seed, offset + 2) if rht else None

    dYq = quantize(dY, grouping="row", fmt=grad_fmt, rounding="sr", rht_mask=mask_dx, seed=seed, offset=offset + 0)
    Wt = quantize(dequantize(Wq), grouping="col", fmt="nvfp4", rounding="sr", rht_mask=mask_dx,
                  seed=seed, offset=offset + 1)
    dYt = quantize(dY, grouping="col", fmt=grad_fmt, rounding="sr", rht_mask=mask_dw, seed=seed, offset=offset + 2)
    Xt = quantize(dequantize(Xq), grouping="col", fmt="nvfp4", rounding="sr", rht_mask=mask_dw,
                  seed=seed, offset=offset + 3)
    out = {"dYq": dYq, "Wt": Wt, "dYt": dYt, "Xt": Xt,
           "mask_dx": mask_dx, "mask_dw": mask_dw}
    dX_rest = gemm_nt_f64(dYq, Wt)
    dW_rest = gemm_nt_f64(dYt, Xt)
    if plan is None:
        out["dX"], out["dW"] = dX_rest, dW_rest
        return out
    K = len(plan.rest) + len(plan.outliers)
    W8t = quantize(dequantize(saved["W8"]), grouping="col", fmt="fp8", rounding="sr", rht_mask=mask_dx,
                   seed=seed, offset=offset + 4)
    X8t = quantize(dequantize(saved["X8"]), grouping="col", fmt="fp8", rounding="sr", rht_mask=mask_dw,
                   seed=seed, offset=offset + 5)
    dX = np.zeros((M, K))
    dW = np.zeros((N, K))
    dX[:, plan.rest] = dX_rest
    dW[:, plan.rest] = dW_rest
    dX[:, plan.outliers] = gemm_nt_f64(dYq, W8t)
    dW[:, plan.outliers] = gemm_nt_f64(dYt, X8t)
    out.update({"W8t": W8t, "X8t": X8t, "dX": dX, "dW": dW})
    return out

"""Reference products on quantized operands (oracle; test infrastructure only).

The three products of the linear layer (Y, dX, dW) run on the quantized
operands (TetraJet-v2 technical summary, section 2: NVFP4 for activations,
weights and gradients of every linear layer).  The reference value of
C = A * B^T, with both operands stored "rows x reduction" and grouped along
the reduction dimension, is the fp64 product of the exactly dequantized
operands (q * s * S, or e * S8 for FP8 segments).  Any summation order is an
equally valid result; the HIP path is compared to this within a relative
Frobenius error bound.
"""
from __future__ import annotations

import numpy as np

from .quant import QTensor, dequantize_f64


def gemm_nt_f64(a: QTensor, b: QTensor) -> np.ndarray:
    """C[i, j] = sum_k A[i, k] * B[j, k] in fp64 on exactly dequantized operands."""
    assert a.L == b.L
    return dequantize_f64(a) @ dequantize_f64(b).T


def gemm_nt_bruteforce(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """Triple loop in Python floats (fp64); tiny shapes only."""
    I, K = A.shape
    J, K2 = B.shape
    assert K == K2
    C = np.zeros((I, J))
    for i in range(I):
        for j in range(J):
            acc = 0.0
            for k in range(K):
                acc += float(A[i, k]) * float(B[j, k])
            C[i, j] = acc
    return C


def rel_fro(c: np.ndarray, ref: np.ndarray) -> float:
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(np.asarray(c, dtype=np.float64) - ref)
    return float(num / den) if den > 0 else float(num)

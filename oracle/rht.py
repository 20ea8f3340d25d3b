"""16-wide random Hadamard transform (oracle; test infrastructure only).

The backward pass applies a random Hadamard transform to the operands of the
dX and dW products to spread outlier energy over channels (TetraJet-v2
technical summary, section 2.C).  The pages fix neither the sign vector nor
the normalisation nor the order of operations; the reading taken:

* the transform acts on consecutive 16-element chunks along the reduction
  dimension of the product: y = (1/4) * H16 * D * x, with D = diag(d),
  d_j = -1 iff bit j of a 16-bit sign mask is set;
* H16 is the Sylvester (natural-order) Hadamard matrix; (1/4) H16 D is
  orthogonal, so applying the same transform to both operands along the
  reduction dimension leaves the exact product unchanged;
* fp32 evaluation order: negate, then butterfly stages with h = 1, 2, 4, 8,
  each pairing (i, i+h) for i with (i & h) == 0 into (a + b, a - b), then
  multiply by 0.25.
"""
from __future__ import annotations

import numpy as np


def sign_vector(mask: int) -> np.ndarray:
    return np.array([-1.0 if (mask >> j) & 1 else 1.0 for j in range(16)])


def fwht16_f32(x: np.ndarray, mask: int) -> np.ndarray:
    """Transform the last axis (length 16) of fp32 x with the given sign mask, in fp32."""
    y = np.array(x, dtype=np.float32, copy=True)
    assert y.shape[-1] == 16
    neg = sign_vector(mask) < 0
    y[..., neg] = -y[..., neg]
    h = 1
    while h < 16:
        out = np.empty_like(y)
        for i in range(16):
            if i & h:
                continue
            a = y[..., i]
            b = y[..., i + h]
            out[..., i] = a + b
            out[..., i + h] = a - b
        y = out
        h *= 2
    return (y * np.float32(0.25)).astype(np.float32)


def rht_along_last(x: np.ndarray, mask: int) -> np.ndarray:
    """Apply the transform to every 16-chunk of the last axis (length a multiple of 16)."""
    x = np.asarray(x, dtype=np.float32)
    L = x.shape[-1]
    assert L % 16 == 0
    y = fwht16_f32(x.reshape(x.shape[:-1] + (L // 16, 16)), mask)
    return y.reshape(x.shape)


def rht_matrix_f64(mask: int) -> np.ndarray:
    """(1/4) H16 D as an fp64 matrix, built by transforming unit vectors in fp64."""
    eye = np.eye(16)
    d = sign_vector(mask)
    cols = []
    for j in range(16):
        y = eye[j] * d
        h = 1
        while h < 16:
            out = y.copy()
            for i in range(16):
                if not i & h:
                    out[i], out[i + h] = y[i] + y[i + h], y[i] - y[i + h]
            y = out
            h *= 2
        cols.append(0.25 * y)
    return np.stack(cols, axis=1)

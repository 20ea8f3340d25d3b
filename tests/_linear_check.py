"""Sampled parity check of one linear layer's forward and backward against the oracle.

The oracle computes only what the sampled outputs need, which is exact because
every quantizer group is local: row-grouped outputs depend on their own row,
column-grouped outputs on their own column, and a product entry on one row of
each operand.  Packed operands are compared bit for bit on the sampled rows;
products on sampled rows x columns against the fp64 product of the oracle's
operands: within 1e-3 relative Frobenius for fp32 outputs, and bf16 outputs
within one bf16 ulp.
"""
from __future__ import annotations

import numpy as np

from oracle import gemm as ogemm, philox, quant

import _helpers as H


def row_block_deq(x_rest: np.ndarray, cols: np.ndarray, fmt: str) -> np.ndarray:
    """Dequantized forward (RTN, row-grouped) values of the given columns, all rows: only the
    128-element blocks holding the requested columns are quantized."""
    L = x_rest.shape[1]
    out = np.empty((x_rest.shape[0], len(cols)), np.float32)
    for b in np.unique(cols // 128):
        lo, hi = b * 128, min(b * 128 + 128, L)
        q = quant.nvfp4_quantize_rows(x_rest[:, lo:hi], "rtn") if fmt == "nvfp4" else \
            quant.fp8_quantize_rows(x_rest[:, lo:hi], "rtn")
        deq = quant.dequantize(q)
        sel = np.nonzero(cols // 128 == b)[0]
        out[:, sel] = deq[:, cols[sel] - lo]
    return out


def sample_cols(rng, L, per_block):
    """Columns from the first, the last (possibly partial) and two random 128-blocks of L."""
    nb = -(-L // 128)
    blocks = np.unique(np.concatenate([[0, nb - 1], rng.choice(nb, min(nb, 2), replace=False)]))
    cols = []
    for b in blocks:
        lo, hi = b * 128, min(b * 128 + 128, L)
        cols.append(rng.choice(np.arange(lo, hi), min(per_block, hi - lo), replace=False))
    return np.unique(np.concatenate(cols + [[L - 1]]))


def check_linear_sampled(X, W, dY, plan_idx, seed, offset, gpu, rng, tag=""):
    """X [M, K] and dY [M, N]: fp32 values of the bf16 inputs; W [N, K]: the fp32 masters the forward
    quantized; plan_idx: sorted outlier channels or None.  gpu: dict with the library's results of
    the call: saved (Xq, Wq, X8, W8), ops (dYq, dYt, Wt, Xt, W8t, X8t), Y / dX (bf16 torch), dW (fp32
    torch) and Y32 / dX32 (the same products with fp32 outputs).  Returns the relative Frobenius errors."""
    M, K = X.shape
    N = W.shape[0]
    rows = np.unique(np.concatenate([rng.choice(M, min(M, 48), replace=False), [0, M - 1]]))
    ns = np.unique(np.concatenate([rng.choice(N, min(N, 32), replace=False), [0, N - 1]]))
    rest = np.arange(K) if plan_idx is None else np.setdiff1d(np.arange(K), plan_idx)
    K1, no = len(rest), (0 if plan_idx is None else len(plan_idx))
    X_rest = np.ascontiguousarray(X[:, rest])
    W_rest = np.ascontiguousarray(W[:, rest])
    mdx, mdw = philox.rht_signs(seed, offset + 0), philox.rht_signs(seed, offset + 2)
    saved, ops = gpu["saved"], gpu["ops"]

    # forward: Y[rows, ns]
    Xq_r = H.oracle_rows(X_rest[rows], rows, K1, "nvfp4", "rtn", 0, 0)
    Wq_r = H.oracle_rows(W_rest[ns], ns, K1, "nvfp4", "rtn", 0, 0)
    H.assert_q_equal(saved["Xq"], Xq_r, rows=rows, what=f"{tag} Xq")
    H.assert_q_equal(saved["Wq"], Wq_r, rows=ns, what=f"{tag} Wq")
    Y_ref = ogemm.gemm_nt_f64(Xq_r, Wq_r)
    # backward: dX[rows, ks / O[ko]], dW[ns, ks2 / O[ko2]]
    dYq_r = H.oracle_rows(dY[rows], rows, N, "nvfp4", "sr", seed, offset + 0, mdx)
    H.assert_q_equal(ops["dYq"], dYq_r, rows=rows, what=f"{tag} dYq")
    ks = sample_cols(rng, K1, 12)
    Wt_r = H.oracle_cols(row_block_deq(W_rest, ks, "nvfp4"), ks, K1, "nvfp4", "sr", seed, offset + 1, mdx)
    H.assert_q_equal(ops["Wt"], Wt_r, rows=ks, what=f"{tag} Wt")
    dX_cols, dX_parts = [rest[ks]], [ogemm.gemm_nt_f64(dYq_r, Wt_r)]
    dYt_r = H.oracle_cols(dY[:, ns], ns, N, "nvfp4", "sr", seed, offset + 2, mdw)
    H.assert_q_equal(ops["dYt"], dYt_r, rows=ns, what=f"{tag} dYt")
    ks2 = sample_cols(rng, K1, 12)
    Xt_r = H.oracle_cols(row_block_deq(X_rest, ks2, "nvfp4"), ks2, K1, "nvfp4", "sr", seed, offset + 3, mdw)
    H.assert_q_equal(ops["Xt"], Xt_r, rows=ks2, what=f"{tag} Xt")
    dW_cols, dW_parts = [rest[ks2]], [ogemm.gemm_nt_f64(dYt_r, Xt_r)]
    if no:
        O = np.asarray(plan_idx)
        X_O, W_O = np.ascontiguousarray(X[:, O]), np.ascontiguousarray(W[:, O])
        X8_r = H.oracle_rows(X_O[rows], rows, no, "fp8", "rtn", 0, 0)
        W8_r = H.oracle_rows(W_O[ns], ns, no, "fp8", "rtn", 0, 0)
        H.assert_q_equal(saved["X8"], X8_r, rows=rows, what=f"{tag} X8")
        H.assert_q_equal(saved["W8"], W8_r, rows=ns, what=f"{tag} W8")
        Y_ref = Y_ref + ogemm.gemm_nt_f64(X8_r, W8_r)
        ko = sample_cols(rng, no, 8)
        W8t_r = H.oracle_cols(row_block_deq(W_O, ko, "fp8"), ko, no, "fp8", "sr", seed, offset + 4, mdx)
        H.assert_q_equal(ops["W8t"], W8t_r, rows=ko, what=f"{tag} W8t")
        dX_cols.append(O[ko])
        dX_parts.append(ogemm.gemm_nt_f64(dYq_r, W8t_r))
        ko2 = sample_cols(rng, no, 8)
        X8t_r = H.oracle_cols(row_block_deq(X_O, ko2, "fp8"), ko2, no, "fp8", "sr", seed, offset + 5, mdw)
        H.assert_q_equal(ops["X8t"], X8t_r, rows=ko2, what=f"{tag} X8t")
        dW_cols.append(O[ko2])
        dW_parts.append(ogemm.gemm_nt_f64(dYt_r, X8t_r))

    import torch
    rows_d = torch.from_numpy(rows).to(gpu["Y"].device)
    ns_d = torch.from_numpy(ns).to(gpu["Y"].device)
    cx = np.concatenate(dX_cols)
    cx_d = torch.from_numpy(cx).to(gpu["Y"].device)
    cw = np.concatenate(dW_cols)
    dX_ref = np.concatenate(dX_parts, axis=1)
    dW_ref = np.concatenate(dW_parts, axis=1)
    Y_s = gpu["Y"][rows_d][:, ns_d].cpu()
    Y32_s = gpu["Y32"][rows_d][:, ns_d].cpu().numpy()
    dX_s = gpu["dX"][rows_d][:, cx_d].cpu()
    dX32_s = gpu["dX32"][rows_d][:, cx_d].cpu().numpy()
    dW_s = gpu["dW"][ns_d].cpu().numpy()[:, cw]
    err = {"Y": H.rel_fro(Y32_s, Y_ref), "dX": H.rel_fro(dX32_s, dX_ref), "dW": H.rel_fro(dW_s, dW_ref)}
    assert max(err.values()) <= H.GEMM_TOL, (tag, err)
    assert H.bf16_ulp_ok(Y_s, Y_ref), f"{tag}: Y beyond one bf16 ulp"
    assert H.bf16_ulp_ok(dX_s, dX_ref), f"{tag}: dX beyond one bf16 ulp"
    # fp32 outputs differ from the fp64 product by accumulation order only
    assert max(err.values()) < 1e-4, (tag, err)
    return err

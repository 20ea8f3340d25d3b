"""GPU parity of the linear layer at full workload size (16384 tokens), in the
launch configuration the benchmark times (fp32 masters quantized inside the
forward call, bf16 Y and dX, fp32 dW, caller workspace, RHT on, seed 0).

Workloads: the OLMo-2-70M-style linears (d_model 512, SwiGLU ffn 2048; X
N(0,1) with 0.5% of the channels x32; no outlier plan) and the
OLMo-2-370M-style linears (d_model 1024, ffn 4096; X[t,c] = z * g_c with
lognormal gains sigma 1.5; top-10% channels in FP8 from 8 calibration
batches).  W ~ N(0, 0.02), dY ~ N(0, 0.01).

The oracle computes only what the sampled outputs need, which is exact because
every quantizer group is local: row-grouped outputs depend on their own row,
column-grouped outputs on their own column, and a product row (or a product
entry) on its operand rows.  Packed operands are compared bit for bit on the
sampled rows; products on the sampled rows (Y, dX: all columns) and the sampled
rows x columns (dW) against the fp64 product of the oracle's operands: within
1e-3 relative Frobenius with fp32 outputs, and the benchmark's bf16 outputs within
one bf16 ulp.
"""
import numpy as np
import pytest
import torch

import synthetic
from oracle import calib, gemm as ogemm, philox, quant

import _helpers as H

pytestmark = pytest.mark.gpu

tj2 = pytest.importorskip("bit_fully_quantized_amd")

SEED = 0
CASES = [("70M", s) for s in synthetic.OLMO70M.linears] + [("370M", s) for s in synthetic.OLMO370M.linears]


def _inputs(family, spec, M, case_seed):
    K, N = spec.K, spec.N
    if family == "70M":
        xb = synthetic.acts_with_outliers_bf16((M, K), 1.0, 0.005, 32.0, synthetic.SEED_X + case_seed)
        plan_idx = None
    else:
        gains = synthetic.lognormal_channel_gains(K, 1.5, synthetic.SEED_GAIN + case_seed)
        xb = synthetic.heavy_tailed_acts_bf16(M, gains, synthetic.SEED_X + case_seed)
        batches = (H.bf16_values(synthetic.heavy_tailed_acts_bf16(M // 8, gains, synthetic.SEED_CALIB + 10 * case_seed + b))
                   for b in range(8))
        plan_idx = calib.select_outliers(calib.channel_scores(batches), 0.10)
    W = synthetic.normal_f32((N, K), 0.02, synthetic.SEED_W + case_seed)
    dyb = synthetic.normal_bf16((M, N), 0.01, synthetic.SEED_DY + case_seed)
    return xb, W, dyb, plan_idx


def _row_block_deq(x_rest: np.ndarray, cols: np.ndarray, fmt: str) -> np.ndarray:
    """Dequantized forward (RTN, row-grouped) values of the given compacted columns, all rows.

    Row quantization is local to each 128-element outer block, so only the blocks
    holding the requested columns are quantized."""
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


def _sample_cols(rng, L, per_block):
    """Columns from the first, the last (possibly partial) and two random 128-blocks of L."""
    nb = -(-L // 128)
    blocks = np.unique(np.concatenate([[0, nb - 1], rng.choice(nb, min(nb, 2), replace=False)]))
    cols = []
    for b in blocks:
        lo, hi = b * 128, min(b * 128 + 128, L)
        cols.append(rng.choice(np.arange(lo, hi), min(per_block, hi - lo), replace=False))
    return np.unique(np.concatenate(cols + [[L - 1]]))


@pytest.mark.parametrize("family,spec", CASES, ids=[f"{f}-{s.name}" for f, s in CASES])
def test_linear_full_size_sampled(family, spec):
    M, K, N = 16384, spec.K, spec.N
    case_seed = [s.name for s in synthetic.OLMO370M.linears].index(spec.name)
    offset = 8 * (case_seed + 1)
    xb, W, dyb, plan_idx = _inputs(family, spec, M, case_seed)
    print(f"[fullsize] {family} {spec.name} M={M} K={K} N={N} outliers={0 if plan_idx is None else len(plan_idx)}",
          flush=True)
    rng = np.random.default_rng(100 + case_seed)
    rows = np.unique(np.concatenate([rng.choice(M, 48, replace=False), [0, M - 1]]))
    ns = np.unique(np.concatenate([rng.choice(N, 24, replace=False), [0, N - 1]]))

    # ---------------- GPU, as the benchmark calls it ----------------
    gplan = tj2.OutlierPlan.from_indices(K, plan_idx) if plan_idx is not None else None
    no = 0 if plan_idx is None else len(plan_idx)
    ws = tj2.linear_bwd_workspace(M, N, K, no)
    Y, saved = tj2.linear_fwd(H.bf16_to_device(xb), H.f32_to_device(W), N, plan=gplan, y_dtype=torch.bfloat16)
    dX, dW, ops = tj2.linear_bwd(H.bf16_to_device(dyb), saved, K, seed=SEED, offset=offset, plan=gplan,
                                 dx_dtype=torch.bfloat16, keep_operands=True, workspace=ws)
    rows_d = torch.from_numpy(rows).cuda()
    Y_s, dX_s = Y[rows_d].cpu(), dX[rows_d].cpu()
    dW_s = dW.cpu().numpy()[ns]
    # the same kernels with fp32 outputs, for the relative Frobenius bar (bf16 output rounding alone
    # is about 1.7e-3 of it)
    Y32, _ = tj2.linear_fwd(H.bf16_to_device(xb), H.f32_to_device(W), N, plan=gplan, y_dtype=torch.float32)
    dX32, _, _ = tj2.linear_bwd(H.bf16_to_device(dyb), saved, K, seed=SEED, offset=offset, plan=gplan,
                                dx_dtype=torch.float32, workspace=ws)
    Y32_s, dX32_s = Y32[rows_d].cpu().numpy(), dX32[rows_d].cpu().numpy()
    torch.cuda.synchronize()

    # ---------------- oracle on the samples ----------------
    X = H.bf16_values(xb)
    dY = H.bf16_values(dyb)
    rest = np.arange(K) if plan_idx is None else np.setdiff1d(np.arange(K), plan_idx)
    K1 = len(rest)
    X_rest = np.ascontiguousarray(X[:, rest])
    mdx, mdw = philox.rht_signs(SEED, offset + 0), philox.rht_signs(SEED, offset + 2)

    Xq_r = H.oracle_rows(X_rest[rows], rows, K1, "nvfp4", "rtn", 0, 0)
    Wq = quant.quantize(W[:, rest], grouping="row", rounding="rtn")
    H.assert_q_equal(saved["Xq"], Xq_r, rows=rows, what="Xq")
    H.assert_q_equal(saved["Wq"], Wq, what="Wq")
    Y_ref = ogemm.gemm_nt_f64(Xq_r, Wq)
    dYq_r = H.oracle_rows(dY[rows], rows, N, "nvfp4", "sr", SEED, offset + 0, mdx)
    Wt = quant.quantize(quant.dequantize(Wq), grouping="col", rounding="sr", rht_mask=mdx, seed=SEED,
                        offset=offset + 1)
    H.assert_q_equal(ops["dYq"], dYq_r, rows=rows, what="dYq")
    H.assert_q_equal(ops["Wt"], Wt, what="Wt")
    dX_ref = np.zeros((len(rows), K))
    dX_ref[:, rest] = ogemm.gemm_nt_f64(dYq_r, Wt)

    # dW on sampled rows n and sampled in-feature columns (some NVFP4, some FP8)
    ks = _sample_cols(rng, K1, 12)
    dYt_r = H.oracle_cols(dY[:, ns], ns, N, "nvfp4", "sr", SEED, offset + 2, mdw)
    Xt_r = H.oracle_cols(_row_block_deq(X_rest, ks, "nvfp4"), ks, K1, "nvfp4", "sr", SEED, offset + 3, mdw)
    H.assert_q_equal(ops["dYt"], dYt_r, rows=ns, what="dYt")
    H.assert_q_equal(ops["Xt"], Xt_r, rows=ks, what="Xt")
    cols_w = [rest[ks]]
    dW_parts = [ogemm.gemm_nt_f64(dYt_r, Xt_r)]

    if plan_idx is not None:
        O = np.asarray(plan_idx)
        X_O = np.ascontiguousarray(X[:, O])
        X8_r = H.oracle_rows(X_O[rows], rows, no, "fp8", "rtn", 0, 0)
        W8 = quant.quantize(W[:, O], grouping="row", fmt="fp8", rounding="rtn")
        H.assert_q_equal(saved["X8"], X8_r, rows=rows, what="X8")
        H.assert_q_equal(saved["W8"], W8, what="W8")
        Y_ref = Y_ref + ogemm.gemm_nt_f64(X8_r, W8)
        W8t = quant.quantize(quant.dequantize(W8), grouping="col", fmt="fp8", rounding="sr", rht_mask=mdx,
                             seed=SEED, offset=offset + 4)
        H.assert_q_equal(ops["W8t"], W8t, what="W8t")
        dX_ref[:, O] = ogemm.gemm_nt_f64(dYq_r, W8t)
        ko = _sample_cols(rng, no, 8)
        X8t_r = H.oracle_cols(_row_block_deq(X_O, ko, "fp8"), ko, no, "fp8", "sr", SEED, offset + 5, mdw)
        H.assert_q_equal(ops["X8t"], X8t_r, rows=ko, what="X8t")
        cols_w.append(O[ko])
        dW_parts.append(ogemm.gemm_nt_f64(dYt_r, X8t_r))

    e_y = H.rel_fro(Y32_s, Y_ref)
    e_dx = H.rel_fro(dX32_s, dX_ref)
    cw = np.concatenate(cols_w)
    e_dw = H.rel_fro(dW_s[:, cw], np.concatenate(dW_parts, axis=1))
    print(f"[fullsize] rel_fro Y {e_y:.2e} dX {e_dx:.2e} dW {e_dw:.2e}", flush=True)
    assert e_y <= H.GEMM_TOL and e_dx <= H.GEMM_TOL and e_dw <= H.GEMM_TOL, (e_y, e_dx, e_dw)
    assert H.bf16_ulp_ok(Y_s, Y_ref), "Y beyond one bf16 ulp"
    assert H.bf16_ulp_ok(dX_s, dX_ref), "dX beyond one bf16 ulp"
    # fp32 outputs differ from the fp64 product by accumulation order only
    assert max(e_y, e_dx, e_dw) < 1e-4

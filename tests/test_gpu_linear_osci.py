"""GPU parity of the linear layer forward/backward (with and without static FP8
outlier channels) and of OsciReset, on the single-linear workload
(X 256x512 bf16 N(0,1), W 512x512 fp32 N(0,0.02), dY 256x512 bf16 N(0,1e-2),
Philox seed 0, RHT on, one OsciReset step) and ragged variants."""
import numpy as np
import pytest
import torch

import synthetic
from oracle import calib, gemm as ogemm, linear as olinear, osci as oosci, quant

import _helpers as H

pytestmark = pytest.mark.gpu

tj2 = pytest.importorskip("bit_fully_quantized_amd")


def _linear_inputs(M, N, K, seed):
    xb = synthetic.normal_bf16((M, K), 1.0, seed)
    W = synthetic.normal_f32((N, K), 0.02, seed + 1)
    dyb = synthetic.normal_bf16((M, N), 0.01, seed + 2)
    return xb, W, dyb


def _check_linear(M, N, K, seed, rht, plan_idx=None, offset=0):
    xb, W, dyb = _linear_inputs(M, N, K, seed)
    X, dY = H.bf16_values(xb), H.bf16_values(dyb)
    oplan = olinear.Plan.from_outliers(K, plan_idx) if plan_idx is not None else None
    gplan = tj2.OutlierPlan.from_indices(K, plan_idx) if plan_idx is not None else None
    ref_f = olinear.linear_fwd(X, W, oplan)
    Y, saved = tj2.linear_fwd(H.bf16_to_device(xb), H.f32_to_device(W), N, plan=gplan, y_dtype=torch.float32)
    H.assert_q_equal(saved["Xq"], ref_f["Xq"], what="Xq")
    H.assert_q_equal(saved["Wq"], ref_f["Wq"], what="Wq")
    if oplan is not None:
        H.assert_q_equal(saved["X8"], ref_f["X8"], what="X8")
        H.assert_q_equal(saved["W8"], ref_f["W8"], what="W8")
    assert H.rel_fro(Y.cpu().numpy(), ref_f["Y"]) <= 1e-5
    ref_b = olinear.linear_bwd(dY, ref_f, seed=seed, offset=offset, rht=rht, plan=oplan)
    dX, dW, ops = tj2.linear_bwd(H.bf16_to_device(dyb), saved, K, seed=seed, offset=offset, rht=rht, plan=gplan,
                                 dx_dtype=torch.float32, keep_operands=True)
    for name in ["dYq", "dYt", "Wt", "Xt"] + (["W8t", "X8t"] if oplan is not None else []):
        H.assert_q_equal(ops[name], ref_b[name], what=name)
    e_dx = H.rel_fro(dX.cpu().numpy(), ref_b["dX"])
    e_dw = H.rel_fro(dW.cpu().numpy(), ref_b["dW"])
    assert e_dx <= H.GEMM_TOL and e_dw <= H.GEMM_TOL, (e_dx, e_dw)
    assert e_dx < 1e-5 and e_dw < 1e-5
    # bf16 outputs through the same path: one bf16 ulp of the reference
    Yb, _ = tj2.linear_fwd(H.bf16_to_device(xb), H.f32_to_device(W), N, plan=gplan, y_dtype=torch.bfloat16)
    assert H.bf16_ulp_ok(Yb, ref_f["Y"])
    dXb, _, _ = tj2.linear_bwd(H.bf16_to_device(dyb), saved, K, seed=seed, offset=offset, rht=rht, plan=gplan,
                               dx_dtype=torch.bfloat16)
    assert H.bf16_ulp_ok(dXb, ref_b["dX"])


def test_single_linear_config():
    _check_linear(256, 512, 512, seed=0, rht=True)


@pytest.mark.parametrize("M,N,K,rht", [(144, 80, 400, True), (128, 256, 128, False), (16, 16, 16, True)])
def test_linear_ragged(M, N, K, rht):
    _check_linear(M, N, K, seed=M + N, rht=rht, offset=8)


def test_linear_with_outliers():
    K = 512
    outl = calib.select_outliers(np.exp(np.random.default_rng(0).standard_normal(K) * 1.5), 0.1)  # 64 channels
    assert len(outl) == 64
    _check_linear(256, 384, K, seed=3, rht=True, plan_idx=outl, offset=16)


def test_linear_long_reduction_split_k():
    """M = 2048 tokens: the dW products (reduction over M) run split over K."""
    K = 512
    outl = calib.select_outliers(np.exp(np.random.default_rng(2).standard_normal(K) * 1.5), 0.1)
    _check_linear(2048, 256, K, seed=5, rht=True, plan_idx=outl, offset=32)


def test_linear_with_outliers_partial_blocks():
    K = 1024
    outl = calib.select_outliers(np.exp(np.random.default_rng(1).standard_normal(K) * 1.5), 0.1)  # 112 channels
    assert len(outl) == 112
    _check_linear(128, 256, K, seed=4, rht=True, plan_idx=outl, offset=24)


@pytest.mark.parametrize("K", [9216, 16896])
def test_linear_wide_rows_with_outliers(K):
    """Rows wider than the forward split kernel stages (fp32 W rows past 32 KB at K = 9216; bf16 X rows
    too at K = 16896): those tensors go through the two gathering row quantizations instead."""
    outl = calib.select_outliers(np.exp(np.random.default_rng(K).standard_normal(K) * 1.5), 0.1)
    _check_linear(32, 64, K, seed=6, rht=True, plan_idx=outl, offset=40)


def _state_to_dev(st):
    return [H.f32_to_device(a) for a in (st.W_prev, st.Q_prev, st.dQ, st.dM)]


def _assert_state(dev, st, W_dev, W_ref):
    for d, r, n in zip(dev, (st.W_prev, st.Q_prev, st.dQ, st.dM), ("W_prev", "Q_prev", "dQ", "dM")):
        np.testing.assert_array_equal(d.cpu().numpy().view(np.uint32), r.view(np.uint32), err_msg=n)
    np.testing.assert_array_equal(W_dev.cpu().numpy().view(np.uint32), W_ref.view(np.uint32), err_msg="W")


@pytest.mark.parametrize("N,K", [(512, 512), (48, 400)])
def test_osci_trajectory(N, K):
    rng = np.random.default_rng(N + K)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    Wd = H.f32_to_device(W)
    dev = [torch.empty_like(Wd) for _ in range(4)]
    wq = tj2.QTensor(tj2.NVFP4, N, K)
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
    tj2.osci_reset_step(Wd, *dev, mode=tj2.OSCI_INIT, Wq_out=wq)
    st, wq_ref = oosci.osci_init(W)
    _assert_state(dev, st, Wd, W)
    H.assert_q_equal(wq, wq_ref, what="init codes")
    # oscillating subset: elements that flip around a bin midpoint every step
    osc = rng.random(W.shape) < 0.05
    total = 0
    for t in range(1, 13):
        step = (rng.standard_normal(W.shape) * 2e-5).astype(np.float32)
        step[osc] = np.where(t % 2, 1, -1) * np.float32(3e-3)
        W = (W + step).astype(np.float32)
        Wd.copy_(H.f32_to_device(W))
        end = t % 6 == 0
        mode = tj2.OSCI_WINDOW_END if end else tj2.OSCI_ACCUM
        tj2.osci_reset_step(Wd, *dev, mode=mode, tau=4.0, reset_enabled=(t >= 6), Wq_out=wq, reset_count=cnt)
        W, st, wq_ref, n = oosci.osci_step(W, st, tau=4.0, window_end=end, reset_enabled=(t >= 6))
        total += n
        _assert_state(dev, st, Wd, W)
        H.assert_q_equal(wq, wq_ref, what=f"codes step {t}")
    assert int(cnt.item()) == total
    assert total > 0


def test_osci_single_linear_config():
    """INIT(W0); W1 = W0 - 1e-4 dW; one WINDOW_END step with resets enabled (tau = 4)."""
    M, N, K = 256, 512, 512
    xb, W0, dyb = _linear_inputs(M, N, K, 0)
    Y, saved = tj2.linear_fwd(H.bf16_to_device(xb), H.f32_to_device(W0), N)
    _, dW, _ = tj2.linear_bwd(H.bf16_to_device(dyb), saved, K, seed=0, offset=0)
    Wd = H.f32_to_device(W0)
    dev = [torch.empty_like(Wd) for _ in range(4)]
    tj2.osci_reset_step(Wd, *dev, mode=tj2.OSCI_INIT)
    st, _ = oosci.osci_init(W0)
    dWh = dW.cpu().numpy()
    W1 = (W0 - np.float32(1e-4) * dWh).astype(np.float32)
    Wd.copy_(H.f32_to_device(W1))
    wq = tj2.QTensor(tj2.NVFP4, N, K)
    tj2.osci_reset_step(Wd, *dev, mode=tj2.OSCI_WINDOW_END, tau=4.0, reset_enabled=True, Wq_out=wq)
    W2, st, wq_ref, n = oosci.osci_step(W1, st, tau=4.0, window_end=True, reset_enabled=True)
    _assert_state(dev, st, Wd, W2)
    H.assert_q_equal(wq, wq_ref, what="codes")


def test_channel_sumsq():
    """fp64 sums in a fixed order: within a few fp64 roundings of the oracle's sums, and the
    same bits on a second run."""
    M, K = 1000, 1024
    gains = synthetic.lognormal_channel_gains(K, 1.5, 5)
    bits = synthetic.heavy_tailed_acts_bf16(M, gains, 6)
    x = H.bf16_to_device(bits)
    acc = torch.zeros(K, dtype=torch.float64, device="cuda")
    tj2.channel_sumsq(x, acc)
    ref = calib.channel_scores([H.bf16_values(bits)])
    np.testing.assert_allclose(acc.cpu().numpy(), ref, rtol=1e-13)
    acc2 = torch.zeros(K, dtype=torch.float64, device="cuda")
    tj2.channel_sumsq(x, acc2)
    assert torch.equal(acc, acc2)


@pytest.mark.parametrize("K,M", [(1024, 2048), (4096, 1024)])
def test_calibrate_plan_equals_oracle(K, M):
    """OutControl calibration through the library (GPU sums over 8 batches, tj2_select_outliers)
    picks exactly the oracle's top 10% channels on the 370M-style heavy-tailed activations."""
    from bit_fully_quantized_amd import outcontrol
    gains = synthetic.lognormal_channel_gains(K, 1.5, 11)
    batches = [synthetic.heavy_tailed_acts_bf16(M, gains, 100 + b) for b in range(8)]
    plan = outcontrol.calibrate([H.bf16_to_device(b) for b in batches], 0.10)
    want = calib.select_outliers(calib.channel_scores([H.bf16_values(b) for b in batches]), 0.10)
    np.testing.assert_array_equal(plan.outliers.cpu().numpy(), want)
    rest = plan.rest.cpu().numpy()
    np.testing.assert_array_equal(np.sort(np.concatenate([want, rest])), np.arange(K))


def test_mfma_peak_probe_result():
    """The measurement helper's MFMA-only loop: every thread's sum is 0.25 * iters exactly."""
    out = torch.full((8 * 256,), -1.0, dtype=torch.float32, device="cuda")
    flops = tj2.mfma_peak_probe(out, 100)
    torch.cuda.synchronize()
    assert flops == 8 * 4 * 100 * 4 * 32768
    assert torch.all(out == 25.0)

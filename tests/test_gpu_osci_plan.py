"""GPU parity of OsciReset and the fused master pass with an OutControl plan (TetraJet-v2 technical
summary, section 2.B with 2.C): Q(w) quantizes the outlier input channels to FP8 and the compacted
rest to NVFP4, as the forward does.  State arrays, masters, codes (NVFP4 rest + FP8 outliers), reset
counts and diagnostics bit-exact against the oracle over trajectories with window-end resets; the
master pass's next-backward operands (W-hat re-grouped along N, SR + RHT) bit-exact against the
oracle's quantizer and equal to what the backward forms itself."""
import numpy as np
import pytest
import torch

from oracle import adamw as oadamw, linear as olinear, osci as oosci, philox, quant

import _helpers as H

pytestmark = pytest.mark.gpu

tj2 = pytest.importorskip("bit_fully_quantized_amd")


def _plans(K, n, seed):
    outl = np.sort(np.random.default_rng(seed).choice(K, size=n, replace=False))
    return olinear.Plan.from_outliers(K, outl), tj2.OutlierPlan.from_indices(K, outl)


def _bits(t):
    return t.cpu().numpy().view(np.uint32)


def _chan(t, oplan):
    """A state array of the library (compacted channel order under a plan: rest channels, then
    outlier channels) in channel order."""
    a = t.cpu().numpy() if isinstance(t, torch.Tensor) else np.asarray(t)
    if oplan is None:
        return a
    out = np.empty_like(a)
    out[:, np.concatenate([oplan.rest, oplan.outliers])] = a
    return out


def _state_bits(t, oplan):
    return _chan(t, oplan).view(np.uint32)


def _check_codes(wq, w8, ref, what):
    H.assert_q_equal(wq, ref[0], what=f"{what} Wq")
    H.assert_q_equal(w8, ref[1], what=f"{what} W8")


@pytest.mark.parametrize("N,K,n", [(96, 400, 48), (256, 1024, 112), (3, 512, 16)])
def test_osci_plan_trajectory(N, K, n):
    rng = np.random.default_rng(N + K + n)
    oplan, gplan = _plans(K, n, N)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[:, oplan.outliers] *= 8.0  # the outlier channels carry larger weights
    Wd = H.f32_to_device(W)
    dev = [torch.empty_like(Wd) for _ in range(4)]
    wq, w8 = tj2.QTensor(tj2.NVFP4, N, K - n), tj2.QTensor(tj2.FP8, N, n)
    flips = torch.zeros(1, dtype=torch.int64, device="cuda")
    hist = torch.zeros(tj2.RISK_BINS, dtype=torch.int64, device="cuda")
    resets = torch.zeros(1, dtype=torch.int64, device="cuda")
    tj2.osci_reset_step(Wd, *dev, mode=tj2.OSCI_INIT, plan=gplan, Wq_out=wq, W8_out=w8)
    st, codes = oosci.osci_init(W, oplan)
    torch.cuda.synchronize()
    _check_codes(wq, w8, codes, "init")
    osc = rng.random(W.shape) < 0.05
    n_reset_total = 0
    for t in range(1, 13):
        step = (rng.standard_normal(W.shape) * 2e-5).astype(np.float32)
        step[osc] = np.where(t % 2, 1, -1) * np.float32(3e-3)
        W = (W + step).astype(np.float32)
        Wd.copy_(H.f32_to_device(W))
        end = t % 6 == 0
        flips.zero_()
        hist.zero_()
        tj2.osci_reset_step(Wd, *dev, mode=tj2.OSCI_WINDOW_END if end else tj2.OSCI_ACCUM, tau=4.0,
                            reset_enabled=t >= 6, plan=gplan, Wq_out=wq, W8_out=w8, reset_count=resets,
                            flips=flips, risk_hist=hist)
        diag = {}
        W, st, codes, nr = oosci.osci_step(W, st, tau=4.0, window_end=end, reset_enabled=t >= 6, diag=diag,
                                           plan=oplan)
        n_reset_total += nr
        torch.cuda.synchronize()
        for d, r, name in zip(dev, (st.W_prev, st.Q_prev, st.dQ, st.dM), ("W_prev", "Q_prev", "dQ", "dM")):
            np.testing.assert_array_equal(_state_bits(d, oplan), r.view(np.uint32), err_msg=f"step {t}: {name}")
        np.testing.assert_array_equal(_bits(Wd), W.view(np.uint32), err_msg=f"step {t}: W")
        _check_codes(wq, w8, codes, f"step {t}")
        assert int(flips.item()) == diag["flips"], f"step {t}: flips"
        if end:
            np.testing.assert_array_equal(hist.cpu().numpy(), diag["risk_hist"], err_msg=f"step {t}: histogram")
    assert int(resets.item()) == n_reset_total > 0


def test_osci_multi_mixed_plans():
    """One multi-matrix call over matrices with and without a plan equals the oracle per matrix."""
    rng = np.random.default_rng(5)
    specs = [(64, 256, 32), (40, 128, 0), (128, 512, 64), (16, 64, 16), (200, 96, 0)]
    mats = []
    for i, (N, K, n) in enumerate(specs):
        W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
        plans = _plans(K, n, i) if n else (None, None)
        Wd = H.f32_to_device(W)
        dev = [torch.empty_like(Wd) for _ in range(4)]
        tj2.osci_reset_step(Wd, *dev, mode=tj2.OSCI_INIT, plan=plans[1])
        st, _ = oosci.osci_init(W, plans[0])
        wq = tj2.QTensor(tj2.NVFP4, N, K - n)
        w8 = tj2.QTensor(tj2.FP8, N, n) if n else None
        mats.append(dict(W=W, Wd=Wd, dev=dev, st=st, plans=plans, wq=wq, w8=w8))
    batch = tj2.OsciBatch([(m["Wd"], *m["dev"], m["wq"], m["plans"][1], m["w8"]) for m in mats])
    for t in range(1, 5):
        for m in mats:
            m["W"] = (m["W"] + (rng.standard_normal(m["W"].shape) * 3e-3).astype(np.float32)).astype(np.float32)
            m["Wd"].copy_(H.f32_to_device(m["W"]))
        end = t == 4
        tj2.osci_reset_step_multi(batch, mode=tj2.OSCI_WINDOW_END if end else tj2.OSCI_ACCUM, tau=1.0,
                                  reset_enabled=True)
        torch.cuda.synchronize()
        for i, m in enumerate(mats):
            m["W"], m["st"], codes, _ = oosci.osci_step(m["W"], m["st"], tau=1.0, window_end=end, reset_enabled=True,
                                                        plan=m["plans"][0])
            np.testing.assert_array_equal(_bits(m["Wd"]), m["W"].view(np.uint32), err_msg=f"{i} step {t}: W")
            np.testing.assert_array_equal(_state_bits(m["dev"][2], m["plans"][0]), m["st"].dQ.view(np.uint32),
                                          err_msg=f"{i}: dQ")
            if m["w8"] is not None:
                _check_codes(m["wq"], m["w8"], codes, f"matrix {i} step {t}")
            else:
                H.assert_q_equal(m["wq"], codes, what=f"matrix {i} step {t}")


@pytest.mark.parametrize("N,K,n", [(256, 1024, 112), (96, 400, 48), (64, 256, 0)])
def test_master_plan_and_next_backward_operands(N, K, n):
    rng = np.random.default_rng(3 * N + K)
    oplan, gplan = _plans(K, n, K) if n else (None, None)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    Wd = H.f32_to_device(W)
    W_prev, Q_prev, dQ, dM = (torch.empty_like(Wd) for _ in range(4))
    m, v = torch.zeros_like(Wd), torch.zeros_like(Wd)
    tj2.osci_reset_step(Wd, W_prev, Q_prev, dQ, dM, mode=tj2.OSCI_INIT, plan=gplan)
    st, _ = oosci.osci_init(W, oplan)
    mo, vo = np.zeros_like(W), np.zeros_like(W)
    opt = oadamw.AdamW(lr=2e-3)
    K1 = K - n
    wq = tj2.QTensor(tj2.NVFP4, N, K1)
    w8 = tj2.QTensor(tj2.FP8, N, n) if n else None
    nxt = tj2.NextBwd(tj2.QTensor(tj2.NVFP4, K1, N), tj2.QTensor(tj2.FP8, n, N) if n else None, seed=7, offset=0)
    osc = rng.random(W.shape) < 0.05
    resets = torch.zeros(1, dtype=torch.int64, device="cuda")
    n_reset_total = 0
    for t in range(1, 9):
        g = (rng.standard_normal(W.shape) * 1e-3).astype(np.float32)
        g[osc] = np.float32(np.where(t % 2, 1.0, -1.0) * 1e-2)
        bc1, bc2 = opt.bias_corrections(t)
        end = t % 4 == 0
        nxt.offset = 8 * t + 16  # the slot of the next backward call
        tj2.master_update_step(Wd, m, v, H.f32_to_device(g), Q_prev, dQ, dM, lr=opt.lr, bias_correction1=float(bc1),
                               bias_correction2=float(bc2), mode=tj2.OSCI_WINDOW_END if end else tj2.OSCI_ACCUM,
                               tau=0.5, reset_enabled=t >= 4, plan=gplan, Wq_out=wq, W8_out=w8, next_bwd=nxt,
                               reset_count=resets)
        W, mo, vo, Qp, dQo, dMo, codes, nr = oadamw.master_step(W, mo, vo, g, st.Q_prev, st.dQ, st.dM, opt, bc1, bc2,
                                                                 tau=0.5, window_end=end, reset_enabled=t >= 4,
                                                                 plan=oplan)
        n_reset_total += nr
        st = oosci.OsciState(W, Qp, dQo, dMo)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(_bits(Wd), W.view(np.uint32), err_msg=f"step {t}: W")
        for name, got, ref in (("m", m, mo), ("v", v, vo), ("Q_prev", Q_prev, Qp), ("dQ", dQ, dQo), ("dM", dM, dMo)):
            np.testing.assert_array_equal(_state_bits(got, oplan), ref.view(np.uint32), err_msg=f"step {t}: {name}")
        if n:
            _check_codes(wq, w8, codes, f"step {t}")
            ref_wq, ref_w8 = codes
        else:
            H.assert_q_equal(wq, codes, what=f"step {t}")
            ref_wq, ref_w8 = codes, None
        # next backward's operands: the oracle's re-grouping of the dequantized forward weights
        mask = philox.rht_signs(7, nxt.offset)
        ref_wt = quant.quantize(quant.dequantize(ref_wq), grouping="col", fmt="nvfp4", rounding="sr", rht_mask=mask,
                                seed=7, offset=nxt.offset + 1)
        H.assert_q_equal(nxt.Wt, ref_wt, what=f"step {t} Wt")
        if n:
            ref_w8t = quant.quantize(quant.dequantize(ref_w8), grouping="col", fmt="fp8", rounding="sr", rht_mask=mask,
                                     seed=7, offset=nxt.offset + 4)
            H.assert_q_equal(nxt.W8t, ref_w8t, what=f"step {t} W8t")
    assert int(resets.item()) == n_reset_total


def test_backward_with_given_weight_operands():
    """nvfp4_linear_bwd with w_given reads the master pass's operands and gives bit-identical dX, dW."""
    M, N, K, n = 512, 256, 1024, 112
    rng = np.random.default_rng(1)
    oplan, gplan = _plans(K, n, 2)
    W = H.f32_to_device((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    X = torch.randn(M, K, device="cuda").to(torch.bfloat16)
    dY = (torch.randn(M, N, device="cuda") * 0.01).to(torch.bfloat16)
    state = [torch.empty_like(W) for _ in range(3)]
    m, v = torch.zeros_like(W), torch.zeros_like(W)
    W_prev = torch.empty_like(W)
    tj2.osci_reset_step(W, W_prev, *state, mode=tj2.OSCI_INIT, plan=gplan)
    wq, w8 = tj2.QTensor(tj2.NVFP4, N, K - n), tj2.QTensor(tj2.FP8, N, n)
    nxt = tj2.NextBwd(tj2.QTensor(tj2.NVFP4, K - n, N), tj2.QTensor(tj2.FP8, n, N), seed=3, offset=40)
    g = torch.randn_like(W) * 1e-3
    tj2.master_update_step(W, m, v, g, *state, lr=1e-3, bias_correction1=0.1, bias_correction2=0.05, plan=gplan,
                           Wq_out=wq, W8_out=w8, next_bwd=nxt)
    _, saved = tj2.linear_fwd(X, None, N, Wq=wq, W8=w8, plan=gplan, y_dtype=torch.float32)
    dX0, dW0, ops0 = tj2.linear_bwd(dY, saved, K, seed=3, offset=40, plan=gplan, dx_dtype=torch.float32,
                                    keep_operands=True)
    ops = tj2.bwd_operands(M, N, K, gplan)
    ops["Wt"], ops["W8t"] = nxt.Wt, nxt.W8t
    dX1, dW1, _ = tj2.linear_bwd(dY, saved, K, seed=3, offset=40, plan=gplan, dx_dtype=torch.float32, operands=ops,
                                 w_given=True)
    torch.cuda.synchronize()
    for a, b, name in ((ops0["Wt"].codes, nxt.Wt.codes, "Wt"), (ops0["W8t"].codes, nxt.W8t.codes, "W8t"),
                       (dX0, dX1, "dX"), (dW0, dW1, "dW")):
        assert torch.equal(a, b), name

"""GPU parity of the oscillation diagnostics (TetraJet-v2 technical summary,
sections 1 and 2.B): per-call flip counts and window-end risk histograms of
osci_reset_step and master_update_step equal the oracle's exactly, and the
state, masters and codes stay bit-exact with the diagnostics switched on.
Shapes cover several workgroups, a ragged K and a last workgroup with lanes
past the final row."""
import numpy as np
import pytest
import torch

from oracle import adamw as oadamw, osci as oosci

import _helpers as H

pytestmark = pytest.mark.gpu

tj2 = pytest.importorskip("bit_fully_quantized_amd")


def _counters():
    return (torch.zeros(1, dtype=torch.int64, device="cuda"),
            torch.zeros(tj2.RISK_BINS, dtype=torch.int64, device="cuda"))


@pytest.mark.parametrize("N,K", [(512, 512), (48, 400), (3, 400), (1024, 1024)])
def test_osci_diag_trajectory(N, K):
    rng = np.random.default_rng(11 * N + K)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    Wd = H.f32_to_device(W)
    dev = [torch.empty_like(Wd) for _ in range(4)]
    wq = tj2.QTensor(tj2.NVFP4, N, K)
    flips, hist = _counters()
    tj2.osci_reset_step(Wd, *dev, mode=tj2.OSCI_INIT, Wq_out=wq, flips=flips, risk_hist=hist)
    st, _ = oosci.osci_init(W)
    torch.cuda.synchronize()
    assert int(flips.item()) == 0 and int(hist.sum().item()) == 0  # INIT counts nothing
    osc = rng.random(W.shape) < 0.05      # flips around a bin midpoint every step
    frozen = rng.random(W.shape) < 0.3    # never moves (dM = 0; dQ > 0 only through its group's scale)
    seen_flips = 0
    for t in range(1, 13):
        step = (rng.standard_normal(W.shape) * 2e-5).astype(np.float32)
        step[osc] = np.where(t % 2, 1, -1) * np.float32(3e-3)
        step[frozen] = 0
        W = (W + step).astype(np.float32)
        Wd.copy_(H.f32_to_device(W))
        end = t % 6 == 0
        mode = tj2.OSCI_WINDOW_END if end else tj2.OSCI_ACCUM
        flips.zero_()
        hist.zero_()
        tj2.osci_reset_step(Wd, *dev, mode=mode, tau=4.0, reset_enabled=(t >= 6), Wq_out=wq, flips=flips,
                            risk_hist=hist)
        diag = {}
        W, st, wq_ref, _ = oosci.osci_step(W, st, tau=4.0, window_end=end, reset_enabled=(t >= 6), diag=diag)
        torch.cuda.synchronize()
        assert int(flips.item()) == diag["flips"], f"step {t}: flips"
        seen_flips += diag["flips"]
        if end:
            np.testing.assert_array_equal(hist.cpu().numpy(), diag["risk_hist"], err_msg=f"step {t}: histogram")
            assert int(hist.sum().item()) == N * K
        else:
            assert int(hist.sum().item()) == 0
        for d, r, n in zip(dev, (st.W_prev, st.Q_prev, st.dQ, st.dM), ("W_prev", "Q_prev", "dQ", "dM")):
            np.testing.assert_array_equal(d.cpu().numpy().view(np.uint32), r.view(np.uint32), err_msg=f"{t}: {n}")
        np.testing.assert_array_equal(Wd.cpu().numpy().view(np.uint32), W.view(np.uint32), err_msg=f"{t}: W")
        H.assert_q_equal(wq, wq_ref, what=f"codes step {t}")
    assert seen_flips > 0


@pytest.mark.parametrize("N,K", [(256, 512), (100, 400)])
def test_master_diag_trajectory(N, K):
    rng = np.random.default_rng(13 * N + K)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    Wd = H.f32_to_device(W)
    W_prev, Q_prev, dQ, dM = (torch.empty_like(Wd) for _ in range(4))
    m, v = torch.zeros_like(Wd), torch.zeros_like(Wd)
    tj2.osci_reset_step(Wd, W_prev, Q_prev, dQ, dM, mode=tj2.OSCI_INIT)
    st, _ = oosci.osci_init(W)
    mo, vo = np.zeros_like(W), np.zeros_like(W)
    opt = oadamw.AdamW(lr=2e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
    wq = tj2.QTensor(tj2.NVFP4, N, K)
    flips, hist = _counters()
    osc = rng.random(W.shape) < 0.05
    for t in range(1, 9):
        g = (rng.standard_normal(W.shape) * 1e-3).astype(np.float32)
        g[osc] = np.float32(np.where(t % 2, 1.0, -1.0) * 1e-2)
        bc1, bc2 = opt.bias_corrections(t)
        end = t % 4 == 0
        mode = tj2.OSCI_WINDOW_END if end else tj2.OSCI_ACCUM
        flips.zero_()
        hist.zero_()
        tj2.master_update_step(Wd, m, v, H.f32_to_device(g), Q_prev, dQ, dM, lr=opt.lr,
                               bias_correction1=float(bc1), bias_correction2=float(bc2), beta1=opt.beta1,
                               beta2=opt.beta2, eps=opt.eps, weight_decay=opt.weight_decay, mode=mode, tau=0.5,
                               reset_enabled=(t >= 4), Wq_out=wq, flips=flips, risk_hist=hist)
        diag = {}
        W, mo, vo, Qp, dQo, dMo, wq_ref, _ = oadamw.master_step(W, mo, vo, g, st.Q_prev, st.dQ, st.dM, opt, bc1, bc2,
                                                                 tau=0.5, window_end=end, reset_enabled=(t >= 4),
                                                                 diag=diag)
        st = oosci.OsciState(W, Qp, dQo, dMo)
        torch.cuda.synchronize()
        assert int(flips.item()) == diag["flips"], f"step {t}: flips"
        if end:
            np.testing.assert_array_equal(hist.cpu().numpy(), diag["risk_hist"], err_msg=f"step {t}: histogram")
        else:
            assert int(hist.sum().item()) == 0
        for name, got, ref in (("W", Wd, W), ("m", m, mo), ("v", v, vo), ("Q_prev", Q_prev, Qp), ("dQ", dQ, dQo),
                               ("dM", dM, dMo)):
            np.testing.assert_array_equal(got.cpu().numpy().view(np.uint32), ref.view(np.uint32),
                                          err_msg=f"step {t}: {name}")
        H.assert_q_equal(wq, wq_ref, what=f"codes step {t}")

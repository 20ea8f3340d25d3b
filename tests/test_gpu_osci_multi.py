"""GPU parity of osci_reset_step_multi (TetraJet-v2 technical summary, section
2.B): twenty weight matrices of mixed shapes (two launches of the multi-problem
kernel, ragged K, rows that end mid-workgroup, with and without codes output)
driven through a multi-step trajectory with a window end and resets; every
state array, master and code bit-exact against the oracle's OsciReset on each
matrix, and the reset count, flip count and risk histogram equal to the
oracle's sums over the matrices."""
import numpy as np
import pytest
import torch

from oracle import osci as oosci

import _helpers as H

pytestmark = pytest.mark.gpu

tj2 = pytest.importorskip("bit_fully_quantized_amd")

SHAPES = [(16, 128), (48, 400), (3, 400), (100, 256), (33, 2048), (64, 16), (1, 128), (130, 144), (17, 912),
          (256, 512), (8, 1040), (40, 96), (5, 4096), (77, 208), (2, 32), (64, 640), (90, 112), (11, 3680),
          (128, 128), (31, 272)]


def test_osci_multi_trajectory():
    rng = np.random.default_rng(21)
    Ws = [(rng.standard_normal(s) * 0.02).astype(np.float32) for s in SHAPES]
    dev = []
    for i, W in enumerate(Ws):
        Wd = H.f32_to_device(W)
        st = [torch.empty_like(Wd) for _ in range(4)]
        wq = tj2.QTensor(tj2.NVFP4, *W.shape) if i % 3 != 1 else None
        dev.append((Wd, *st, wq))
    tj2.osci_reset_step_multi(dev, mode=tj2.OSCI_INIT)
    states = [oosci.osci_init(W)[0] for W in Ws]
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
    flips = torch.zeros(1, dtype=torch.int64, device="cuda")
    hist = torch.zeros(tj2.RISK_BINS, dtype=torch.int64, device="cuda")
    osc = [rng.random(s) < 0.05 for s in SHAPES]
    total_resets = 0
    for t in range(1, 7):
        end = t == 6
        for i, W in enumerate(Ws):
            step = (rng.standard_normal(W.shape) * 2e-5).astype(np.float32)
            step[osc[i]] = np.where(t % 2, 1, -1) * np.float32(3e-3)
            Ws[i] = (W + step).astype(np.float32)
            dev[i][0].copy_(H.f32_to_device(Ws[i]))
        flips.zero_()
        hist.zero_()
        tj2.osci_reset_step_multi(dev, mode=tj2.OSCI_WINDOW_END if end else tj2.OSCI_ACCUM, tau=4.0,
                                  reset_enabled=end, reset_count=cnt, flips=flips, risk_hist=hist)
        want_flips, want_hist = 0, np.zeros(tj2.RISK_BINS, np.int64)
        for i in range(len(Ws)):
            diag = {}
            Ws[i], states[i], wq_ref, n_reset = oosci.osci_step(Ws[i], states[i], tau=4.0, window_end=end,
                                                                reset_enabled=end, diag=diag)
            total_resets += n_reset
            want_flips += diag["flips"]
            if end:
                want_hist += diag["risk_hist"]
            Wd, Wp, Qp, dQ, dM, wq = dev[i]
            st = states[i]
            for d, r, n in ((Wd, Ws[i], "W"), (Wp, st.W_prev, "W_prev"), (Qp, st.Q_prev, "Q_prev"), (dQ, st.dQ, "dQ"),
                            (dM, st.dM, "dM")):
                np.testing.assert_array_equal(d.cpu().numpy().view(np.uint32), r.view(np.uint32),
                                              err_msg=f"step {t}, matrix {i} {SHAPES[i]}: {n}")
            if wq is not None:
                H.assert_q_equal(wq, wq_ref, what=f"step {t}, matrix {i} codes")
        torch.cuda.synchronize()
        assert int(flips.item()) == want_flips, f"step {t}: flips"
        np.testing.assert_array_equal(hist.cpu().numpy(), want_hist, err_msg=f"step {t}: histogram")
    assert total_resets > 0 and int(cnt.item()) == total_resets


def test_master_multi_trajectory():
    """master_update_step_multi (fused AdamW + OsciReset + codes, section 2.B) on eighteen matrices: every
    master, moment, state array and code bit-exact against the oracle's master step per matrix."""
    from oracle import adamw as oadamw
    shapes = SHAPES[:18]
    rng = np.random.default_rng(23)
    Ws = [(rng.standard_normal(s) * 0.02).astype(np.float32) for s in shapes]
    opt = oadamw.AdamW(lr=2e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
    dev, ref = [], []
    for i, W in enumerate(Ws):
        Wd = H.f32_to_device(W)
        Qp, dQ, dM = (torch.empty_like(Wd) for _ in range(3))
        tj2.osci_reset_step(Wd, torch.empty_like(Wd), Qp, dQ, dM, mode=tj2.OSCI_INIT)
        g = torch.empty_like(Wd)
        wq = tj2.QTensor(tj2.NVFP4, *W.shape) if i % 3 != 2 else None
        dev.append([Wd, torch.zeros_like(Wd), torch.zeros_like(Wd), g, Qp, dQ, dM, wq])
        st = oosci.osci_init(W)[0]
        ref.append([W, np.zeros_like(W), np.zeros_like(W), st.Q_prev, st.dQ, st.dM])
    batch = tj2.MasterBatch(dev)
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
    flips = torch.zeros(1, dtype=torch.int64, device="cuda")
    hist = torch.zeros(tj2.RISK_BINS, dtype=torch.int64, device="cuda")
    osc = [rng.random(s) < 0.05 for s in shapes]
    total_resets = 0
    for t in range(1, 5):
        end = t == 4
        grads = []
        for i, s in enumerate(shapes):
            gr = (rng.standard_normal(s) * 1e-3).astype(np.float32)
            gr[osc[i]] = np.float32(np.where(t % 2, 1.0, -1.0) * 1e-2)
            dev[i][3].copy_(H.f32_to_device(gr))
            grads.append(gr)
        bc1, bc2 = opt.bias_corrections(t)
        flips.zero_()
        hist.zero_()
        tj2.master_update_step_multi(batch, lr=opt.lr, bias_correction1=float(bc1), bias_correction2=float(bc2),
                                     beta1=opt.beta1, beta2=opt.beta2, eps=opt.eps, weight_decay=opt.weight_decay,
                                     mode=tj2.OSCI_WINDOW_END if end else tj2.OSCI_ACCUM, tau=0.5, reset_enabled=end,
                                     reset_count=cnt, flips=flips, risk_hist=hist)
        want_flips, want_hist = 0, np.zeros(tj2.RISK_BINS, np.int64)
        for i in range(len(shapes)):
            W, mo, vo, Qp, dQo, dMo = ref[i]
            diag = {}
            W, mo, vo, Qp, dQo, dMo, wq_ref, n_reset = oadamw.master_step(W, mo, vo, grads[i], Qp, dQo, dMo, opt,
                                                                          bc1, bc2, tau=0.5, window_end=end,
                                                                          reset_enabled=end, diag=diag)
            ref[i] = [W, mo, vo, Qp, dQo, dMo]
            total_resets += n_reset
            want_flips += diag["flips"]
            if end:
                want_hist += diag["risk_hist"]
            Wd, m, v, _, Qd, dQd, dMd, wq = dev[i]
            for name, got, r in (("W", Wd, W), ("m", m, mo), ("v", v, vo), ("Q_prev", Qd, Qp), ("dQ", dQd, dQo),
                                 ("dM", dMd, dMo)):
                np.testing.assert_array_equal(got.cpu().numpy().view(np.uint32), r.view(np.uint32),
                                              err_msg=f"step {t}, matrix {i} {shapes[i]}: {name}")
            if wq is not None:
                H.assert_q_equal(wq, wq_ref, what=f"step {t}, matrix {i} codes")
        torch.cuda.synchronize()
        assert int(flips.item()) == want_flips, f"step {t}: flips"
        np.testing.assert_array_equal(hist.cpu().numpy(), want_hist, err_msg=f"step {t}: histogram")
    assert int(cnt.item()) == total_resets

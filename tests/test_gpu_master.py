"""GPU parity of the fused master-weight pass (AdamW, then OsciReset with the
pre-update master as W_prev, then the forward codes): every state array and the
codes bit-exact against the oracle over a trajectory of steps with a window end
and resets, on a full-block and a ragged shape."""
import numpy as np
import pytest
import torch

from oracle import adamw as oadamw, osci as oosci

import _helpers as H

pytestmark = pytest.mark.gpu

tj2 = pytest.importorskip("bit_fully_quantized_amd")


@pytest.mark.parametrize("N,K", [(256, 512), (100, 400)])
def test_master_trajectory(N, K):
    rng = np.random.default_rng(7 * N + K)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    Wd = H.f32_to_device(W)
    W_prev, Q_prev, dQ, dM = (torch.empty_like(Wd) for _ in range(4))
    m = torch.zeros_like(Wd)
    v = torch.zeros_like(Wd)
    tj2.osci_reset_step(Wd, W_prev, Q_prev, dQ, dM, mode=tj2.OSCI_INIT)
    st, _ = oosci.osci_init(W)
    mo, vo = np.zeros_like(W), np.zeros_like(W)
    opt = oadamw.AdamW(lr=2e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
    wq = tj2.QTensor(tj2.NVFP4, N, K)
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
    total = 0
    osc = rng.random(W.shape) < 0.05  # gradients that flip sign every step
    for t in range(1, 9):
        g = (rng.standard_normal(W.shape) * 1e-3).astype(np.float32)
        g[osc] = np.float32(np.where(t % 2, 1.0, -1.0) * 1e-2)
        bc1, bc2 = opt.bias_corrections(t)
        end = t % 4 == 0
        mode = tj2.OSCI_WINDOW_END if end else tj2.OSCI_ACCUM
        tj2.master_update_step(Wd, m, v, H.f32_to_device(g), Q_prev, dQ, dM, lr=opt.lr,
                               bias_correction1=float(bc1), bias_correction2=float(bc2), beta1=opt.beta1,
                               beta2=opt.beta2, eps=opt.eps, weight_decay=opt.weight_decay, mode=mode, tau=0.5,
                               reset_enabled=(t >= 4), Wq_out=wq, reset_count=cnt)
        W, mo, vo, Qp, dQo, dMo, wq_ref, n = oadamw.master_step(W, mo, vo, g, st.Q_prev, st.dQ, st.dM, opt, bc1,
                                                                 bc2, tau=0.5, window_end=end,
                                                                 reset_enabled=(t >= 4))
        st = oosci.OsciState(W, Qp, dQo, dMo)
        total += n
        for name, got, ref in (("W", Wd, W), ("m", m, mo), ("v", v, vo), ("Q_prev", Q_prev, Qp), ("dQ", dQ, dQo),
                               ("dM", dM, dMo)):
            np.testing.assert_array_equal(got.cpu().numpy().view(np.uint32), ref.view(np.uint32),
                                          err_msg=f"step {t}: {name}")
        H.assert_q_equal(wq, wq_ref, what=f"codes step {t}")
    torch.cuda.synchronize()
    assert int(cnt.item()) == total
    assert total > 0

"""Pins of the oracle's AdamW step and fused master-weight pass (CPU only).

The step is pinned against an independent implementation (torch.optim.AdamW on
the CPU, whose operation order differs, so agreement is within fp32 rounding of
the update), against closed forms (zero gradient: decay only; first step with
zero moments and no decay: u = g / (|g| + eps) up to rounding), and the fused
pass against the composition of its pinned parts."""
import numpy as np
import pytest
import torch

from oracle import adamw, osci

EPS32 = np.float32(2.0 ** -24)


def _rand(shape, seed, scale):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


@pytest.mark.parametrize("wd", [0.0, 0.1])
def test_against_torch_adamw(wd):
    W0 = _rand((64, 96), 1, 0.02)
    opt = adamw.AdamW(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=wd)
    W, m, v = W0.copy(), np.zeros_like(W0), np.zeros_like(W0)
    Wt = torch.tensor(W0.copy(), requires_grad=True)
    ot = torch.optim.AdamW([Wt], lr=1e-3, betas=(0.9, 0.95), eps=1e-8, weight_decay=wd)
    for t in range(1, 6):
        g = _rand(W0.shape, 10 + t, 1e-3)
        bc1, bc2 = opt.bias_corrections(t)
        Wp, mp, vp = W.copy(), m.copy(), v.copy()
        W, m, v = adamw.adamw_step(W, m, v, g, opt, bc1, bc2)
        Wt.grad = torch.tensor(g)
        ot.step()
        st = ot.state[Wt]
        Wr, mr, vr = Wt.detach().numpy(), st["exp_avg"].numpy(), st["exp_avg_sq"].numpy()
        # agreement within fp32 rounding: of the values m and v are formed from, and for W of the
        # previous master plus 1e-4 of the update (the two compute the update in different orders;
        # a wrong term, sign or bias correction is off by a sizeable fraction of the update)
        assert np.all(np.abs(W - Wr) <= 4 * EPS32 * np.abs(Wp) + 1e-4 * np.abs(W - Wp) + 1e-30), t
        assert np.all(np.abs(m - mr) <= 8 * EPS32 * (0.9 * np.abs(mp) + 0.1 * np.abs(g)) + 1e-30), t
        assert np.all(np.abs(v - vr) <= 8 * EPS32 * (0.95 * vp + 0.05 * g * g) + 1e-38), t
        # both continue from the oracle's state
        Wt.data.copy_(torch.tensor(W))
        st["exp_avg"].copy_(torch.tensor(m))
        st["exp_avg_sq"].copy_(torch.tensor(v))


def test_zero_gradient_is_pure_decay():
    W = _rand((32, 48), 2, 0.02)
    opt = adamw.AdamW(lr=3e-4, weight_decay=0.1)
    bc1, bc2 = opt.bias_corrections(7)
    z = np.zeros_like(W)
    W1, m1, v1 = adamw.adamw_step(W, z, z, z, opt, bc1, bc2)
    decay = np.float32(np.float32(1.0) - np.float32(np.float32(3e-4) * np.float32(0.1)))
    np.testing.assert_array_equal(W1, (W * decay).astype(np.float32))
    assert not m1.any() and not v1.any()


def test_first_step_closed_form():
    W = _rand((16, 64), 3, 0.02)
    g = _rand(W.shape, 4, 1e-2)
    opt = adamw.AdamW(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.0)
    bc1, bc2 = opt.bias_corrections(1)
    W1, m1, v1 = adamw.adamw_step(W, np.zeros_like(W), np.zeros_like(W), g, opt, bc1, bc2)
    g64 = g.astype(np.float64)
    ref = W.astype(np.float64) - 1e-3 * g64 / (np.abs(g64) + 1e-8)
    assert np.all(np.abs(W1 - ref) <= 8 * EPS32 * (np.abs(W) + 1e-3))
    np.testing.assert_allclose(m1, 0.1 * g64, rtol=3e-7)
    np.testing.assert_allclose(v1, 0.05 * g64 * g64, rtol=5e-7)


def test_bias_corrections():
    opt = adamw.AdamW(lr=1e-3, beta1=0.9, beta2=0.95)
    bc1, bc2 = opt.bias_corrections(1)
    assert bc1 == np.float32(0.1) and bc2 == np.float32(1.0 - 0.95)
    bc1, bc2 = opt.bias_corrections(10 ** 6)
    assert bc1 == np.float32(1.0) and bc2 == np.float32(1.0)


def test_master_step_is_adamw_then_osci():
    W = _rand((24, 256), 5, 0.02)
    st, _ = osci.osci_init(W)
    m = np.zeros_like(W)
    v = np.zeros_like(W)
    opt = adamw.AdamW(lr=1e-2)
    for t in range(1, 5):
        g = _rand(W.shape, 20 + t, 1e-3)
        bc1, bc2 = opt.bias_corrections(t)
        end = t == 4
        W2, m2, v2, Qp, dQ, dM, Wq, n = adamw.master_step(W, m, v, g, st.Q_prev, st.dQ, st.dM, opt, bc1, bc2,
                                                         tau=0.5, window_end=end, reset_enabled=True)
        W1, m1, v1 = adamw.adamw_step(W, m, v, g, opt, bc1, bc2)
        W2r, st2, Wqr, nr = osci.osci_step(W1, osci.OsciState(W.copy(), st.Q_prev, st.dQ, st.dM), 0.5, end, True)
        np.testing.assert_array_equal(W2, W2r)
        np.testing.assert_array_equal(dM, st2.dM)
        assert n == nr
        # the master's distance this step is the update itself
        if not end:
            np.testing.assert_array_equal(dM, (st.dM + np.abs(W1 - W)).astype(np.float32))
        W, m, v = W2, m2, v2
        st = osci.OsciState(W2.copy(), Qp, dQ, dM)

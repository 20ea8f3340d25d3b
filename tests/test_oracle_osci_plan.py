"""Pins for OsciReset with an OutControl plan (oracle.osci with `plan`).

TetraJet-v2 technical summary, section 2.B (reset to the centre of the current
quantization bin of the forward quantizer) with section 2.C (the outlier input
channels stay in FP8 in the forward pass).  Values worked by hand: an outlier
block whose largest element is 448 has the FP32 scale 448 / 448 = 1, so its
E4M3 grid near 1 is {1, 1.125} with the rounding boundary at 1.0625.
"""
import numpy as np

from oracle import formats, linear as olinear, osci

f32 = np.float32


def _plan(K, outl):
    return olinear.Plan.from_outliers(K, outl)


def test_q_is_the_forward_quantizer_with_a_plan():
    """Q(w) scatters exactly the dequantized operands the forward multiplies (NVFP4 rest, FP8 outliers)."""
    rng = np.random.default_rng(0)
    N, K = 48, 256
    W = (rng.standard_normal((N, K)) * 0.02).astype(f32)
    W[:, 7] *= 40
    plan = _plan(K, np.arange(0, 256, 16))
    Q, (Wq, W8) = osci.fwd_quant(W, plan)
    fwd = olinear.linear_fwd(np.zeros((16, K), f32), W, plan)
    from oracle.quant import dequantize
    np.testing.assert_array_equal(Q[:, plan.rest], dequantize(fwd["Wq"]))
    np.testing.assert_array_equal(Q[:, plan.outliers], dequantize(fwd["W8"]))
    np.testing.assert_array_equal(Wq.codes, fwd["Wq"].codes)
    np.testing.assert_array_equal(W8.codes, fwd["W8"].codes)


def _oscillating(N=4, K=64):
    # outlier channels 0..15; channel 3 holds the block maximum 448 (FP8 scale exactly 1) and
    # channel 5 oscillates across the E4M3 boundary 1.0625 between 1 and 1.125; rest channel 40
    # oscillates across the E2M1 boundary between 0 and 0.5 of its block (0.25 * d)
    plan = _plan(K, np.arange(16))
    W = np.zeros((N, K), f32)
    W[:, 3] = 448.0
    W[:, 5] = 1.0624
    W[:, 17] = 6.0      # rest block maximum: S = fl(6 / 2688), inner scale 448, so d = fl(448 S) ~ 1
    W[:, 32] = 6.0      # channels 32..47 are the second rest group (compacted positions 16..31)
    W[:, 40] = 0.2499   # in that group, with the same d ~ 1: 0.2499 -> 0, 0.2501 -> 0.5
    return W, plan


def test_outlier_channel_resets_to_its_fp8_point():
    W, plan = _oscillating()
    st, _ = osci.osci_init(W, plan)
    diag = {}
    flips_expected = 0
    for step in range(1, 9):
        W = W.copy()
        W[:, 5] = f32(1.0626) if step % 2 else f32(1.0624)
        W[:, 40] = f32(0.2501) if step % 2 else f32(0.2499)
        flips_expected += 2 * W.shape[0]  # both oscillating elements change bin every step
        end = step == 8
        W, st, (Wq, W8), n = osci.osci_step(W, st, tau=4.0, window_end=end, reset_enabled=True, diag=diag,
                                            plan=plan)
    assert diag["flips"] == flips_expected
    # step 8 leaves channel 5 at 1.0624 -> Q = 1.0 (E4M3), channel 40 at 0.2499 -> Q = 0 (E2M1)
    assert n == 2 * W.shape[0]
    assert np.all(W[:, 5] == f32(1.0)) and np.all(W[:, 40] == f32(0.0))
    # the reset value of the outlier channel is an E4M3 value times the block scale 1
    assert float(W[0, 5]) in set(formats.E4M3_POS.tolist())
    # untouched elements keep their bits
    for c in (3, 17, 32):
        assert np.all(W[:, c] == _oscillating()[0][:, c])
    # re-quantizing the reset masters returns the same codes (the reset point is a fixed point)
    _, (Wq2, W82) = osci.fwd_quant(W, plan)
    np.testing.assert_array_equal(Wq2.codes, Wq.codes)
    np.testing.assert_array_equal(W82.codes, W8.codes)


def test_outlier_reset_differs_from_e2m1_reading():
    """Without the plan the same trajectory quantizes channel 5 on the E2M1 grid of its block
    (maximum 448: S = 1/6, inner scale 448 -> d = 74.67), where 1.06 rounds to 0: the plan-free
    reading would reset the outlier weight to 0, the plan-aware one keeps it at its FP8 point."""
    W, plan = _oscillating()
    Qp, _ = osci.fwd_quant(W, plan)
    Qn, _ = osci.fwd_quant(W, None)
    assert Qp[0, 5] == f32(1.0) and Qn[0, 5] == f32(0.0)

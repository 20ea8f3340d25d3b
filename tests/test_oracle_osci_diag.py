"""Pins for the oscillation diagnostics of oracle.osci (flip counts, risk histogram).

TetraJet-v2 technical summary, section 1 (weight oscillation: a quantized
weight flips between adjacent bins under small master updates) and section
2.B (the risk dist_Q / dist_M).  References independent of the oracle's code:
the pages' flip example worked by hand (tests/golden/osci_flip_example.json),
a monotone trajectory whose bin crossings are counted by hand on the E2M1
grid, and a per-element brute force of the risk bins with math.frexp.
"""
import math

import numpy as np

from oracle import osci

from test_oracle_osci_calib import flip_trajectory


def run(W0, ws, tau=4.0, reset_enabled=True):
    """Drive element (0, 5) through the values ws (ws[0] at init); one window ending at the last step.
    Returns the per-step flip counts and the window's histogram."""
    st, _ = osci.osci_init(W0)
    Wc = W0
    flips, diag = [], {}
    for t, w in enumerate(ws[1:], start=1):
        Wn = Wc.copy()
        Wn[0, 5] = w
        before = diag.get("flips", 0)
        Wc, st, _, _ = osci.osci_step(Wn, st, tau=tau, window_end=(t == len(ws) - 1), reset_enabled=reset_enabled,
                                      diag=diag)
        flips.append(diag["flips"] - before)
    return flips, diag["risk_hist"]


def test_flip_example_counts():
    W, steps, (lo, hi) = flip_trajectory()
    W0 = W.copy()
    W0[0, 5] = steps[0]
    flips, hist = run(W0, steps)
    # the element alternates between the bins 0 and 0.5 (step d = 1) on every update
    assert flips == [1] * (len(steps) - 1)
    # window: dQ = 49 * 0.5 = 24.5, dM = 49 * 0.002 ~ 0.098 -> risk ~ 250 -> floor(log2) = 7 -> bin 23;
    # every other element never moved (dQ = 0) -> bin 0
    expect = np.zeros(osci.RISK_BINS, np.int64)
    expect[0] = W.size - 1
    expect[16 + 7] = 1
    np.testing.assert_array_equal(hist, expect)


def test_monotone_motion_counts_each_crossing_once():
    W, _, _ = flip_trajectory()
    W0 = W.copy()
    ws = [np.float32(0.1 + 0.05 * t) for t in range(51)]  # 0.1 -> 2.6 in d = 1 units
    W0[0, 5] = ws[0]
    flips, hist = run(W0, ws)
    # round-to-nearest on the E2M1 grid, ties to the even code, written out as thresholds:
    # <= 0.25 -> 0, < 0.75 -> 0.5, <= 1.25 -> 1, < 1.75 -> 1.5, <= 2.5 -> 2, < 3.5 -> 3
    def q(v):
        for bound, inclusive, val in ((0.25, True, 0.0), (0.75, False, 0.5), (1.25, True, 1.0), (1.75, False, 1.5),
                                      (2.5, True, 2.0), (3.5, False, 3.0)):
            if v < bound or (inclusive and v == bound):
                return val
        return 4.0
    crossings = [t for t in range(1, 51) if q(ws[t]) != q(ws[t - 1])]
    assert len(crossings) == 5  # 0 -> 0.5 -> 1 -> 1.5 -> 2 -> 3
    assert [t for t, f in enumerate(flips, start=1) if f] == crossings and sum(flips) == 5
    # dQ = 3 (0 -> 3 monotonically), dM = 2.5 -> risk 1.2 -> bin 16
    assert hist[16] == 1 and hist[0] == W.size - 1 and hist.sum() == W.size


def brute_bin(q, m):
    q, m = np.float32(q), np.float32(m)
    if q == 0:
        return 0
    if m == 0:
        return 31
    with np.errstate(over="ignore", under="ignore"):
        r = float(np.float32(q / m))
    if r == 0.0:
        return 1
    if math.isinf(r):
        return 30
    _, e = math.frexp(r)  # r = f * 2^e with f in [0.5, 1): floor(log2 r) = e - 1
    return min(max(e - 1 + 16, 1), 30)


def test_risk_bins_bruteforce():
    r = np.random.default_rng(3)
    n = 4000
    dQ = (r.random(n) * 10.0 ** r.integers(-8, 8, n)).astype(np.float32)
    dM = (r.random(n) * 10.0 ** r.integers(-8, 8, n)).astype(np.float32)
    dQ[r.random(n) < 0.1] = 0
    dM[r.random(n) < 0.1] = 0
    # exact powers of two and ratios sitting on bin edges
    k = r.integers(-20, 20, 200)
    dQ[:200] = np.ldexp(np.float32(1.0), k).astype(np.float32)
    dM[:200] = 1.0
    dQ[200:210] = np.float32(3e38)
    dM[200:210] = np.float32(1e-38)  # quotient overflows to inf
    dQ[210:220] = np.float32(1e-38)
    dM[210:220] = np.float32(3e38)  # quotient underflows to 0
    got = osci.risk_bin(dQ, dM)
    want = np.array([brute_bin(a, b) for a, b in zip(dQ, dM)])
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(osci.risk_histogram(dQ, dM), np.bincount(want, minlength=32))
    # the power-of-two rows land on the bin of their exponent
    np.testing.assert_array_equal(got[:200], np.clip(k + 16, 1, 30))


def test_histogram_invariants():
    r = np.random.default_rng(4)
    dQ = (r.random((64, 128)) * 0.5 + 0.25).astype(np.float32)
    dM = (r.random((64, 128)) * 0.5 + 0.25).astype(np.float32)
    h = osci.risk_histogram(dQ, dM)
    assert h.sum() == dQ.size
    # doubling dQ (exact) moves every element up by one bin, away from the clamped ends
    h2 = osci.risk_histogram((dQ * 2).astype(np.float32), dM)
    np.testing.assert_array_equal(h2[1:], h[:-1])


def test_scale_drift_is_not_a_flip():
    # Growing a block's largest element moves its FP32 outer scale, and with it the dequantized
    # value of every element of the block, but no element changes bin: no flips.
    r = np.random.default_rng(5)
    W = (r.standard_normal((16, 128)) * 0.02).astype(np.float32)
    W[:, 7] = 0.5  # the largest element of every row's single outer block
    st, _ = osci.osci_init(W)
    W1 = W.copy()
    W1[:, 7] = np.float32(0.5 * (1 + 2 ** -20))
    diag = {}
    _, st1, _, _ = osci.osci_step(W1, st, tau=4.0, window_end=False, reset_enabled=False, diag=diag)
    assert np.count_nonzero(st1.Q_prev != st.Q_prev) > 1000  # the values moved...
    assert diag["flips"] == 0  # ...the bins did not
    # one element pushed across a bin edge is one flip
    W2 = W1.copy()
    q1 = osci.fwd_codes(W1)
    i = int(np.argmax((q1[0] & 7) == 2))  # an element of row 0 at the grid value 1 (in its group's steps)
    W2[0, i] = np.float32(W1[0, i] * 1.6)
    diag = {}
    osci.osci_step(W2, st1, tau=4.0, window_end=False, reset_enabled=False, diag=diag)
    assert diag["flips"] == int(np.count_nonzero(osci.fwd_codes(W2) != q1)) >= 1

"""Pins for oracle.osci (OsciReset) and oracle.calib (OutControl calibration).

Independent references: hand-built trajectories -- the pages' example of a
weight flipping between the adjacent bins 0 and 0.5 around the midpoint 0.25
(tests/golden/osci_flip_example.json; TetraJet-v2 technical summary, sections
1 and 2.B) must be reset to its bin centre, while a steadily moving weight
must be left untouched -- and brute-force top-k for the static outlier set
(section 2.C).
"""
import json
import os

import numpy as np

from oracle import calib, osci, quant

HERE = os.path.dirname(__file__)


def flip_trajectory():
    """A 16x128 weight whose element (0, 5) jitters around the 0 / 0.5 midpoint of its group."""
    ex = json.load(open(os.path.join(HERE, "golden", "osci_flip_example.json")))
    lo, hi = ex["bins"]
    mid = ex["midpoint"]
    assert mid == (lo + hi) / 2
    W = np.zeros((16, 128), np.float32)
    W[:, 0] = 6.0  # each 16-group of row r has max 6 -> s*S chosen so d = 1 in row 0 below
    W[:, 16] = 2688.0  # outer max -> S = 1 in every row; group 0 max 6 -> s = 1 -> d = 1
    eps = np.float32(1e-3)
    steps = [mid - eps, mid + eps] * 25
    return W, steps, (lo, hi)


def test_flip_example_is_reset_to_bin_centre():
    W, steps, (lo, hi) = flip_trajectory()
    W0 = W.copy()
    W0[0, 5] = steps[0]
    st, _ = osci.osci_init(W0)
    Wc = W0
    for t, w in enumerate(steps[1:], start=1):
        Wn = Wc.copy()
        Wn[0, 5] = w
        end = t == len(steps) - 1
        Wc, st, Wq, n = osci.osci_step(Wn, st, tau=4.0, window_end=end, reset_enabled=True)
    # the element flipped 0 <-> 0.5 every step: dQ = 24.5, dM ~ 0.1 -> reset to Q(w)
    assert n == 1
    assert Wc[0, 5] in (lo, hi)
    qv = quant.dequantize(Wq)
    assert qv[0, 5] == Wc[0, 5]
    # everything else untouched
    mask = np.ones_like(Wc, bool)
    mask[0, 5] = False
    np.testing.assert_array_equal(Wc[mask], W0[mask])
    assert np.all(st.dQ == 0) and np.all(st.dM == 0)


def test_steady_motion_not_reset_and_disabled_switch():
    W, _, _ = flip_trajectory()
    W0 = W.copy()
    W0[0, 5] = 0.1
    st, _ = osci.osci_init(W0)
    Wc = W0
    for t in range(1, 51):
        Wn = Wc.copy()
        Wn[0, 5] = np.float32(0.1 + 0.05 * t)  # crosses several bins once, monotonically
        Wc, st, _, n = osci.osci_step(Wn, st, tau=4.0, window_end=(t == 50), reset_enabled=True)
    assert n == 0 and Wc[0, 5] == np.float32(0.1 + 0.05 * 50)
    # flipping weight with the learning-rate switch off: nothing is reset
    W, steps, _ = flip_trajectory()
    W0 = W.copy(); W0[0, 5] = steps[0]
    st, _ = osci.osci_init(W0)
    Wc = W0
    for t, w in enumerate(steps[1:], start=1):
        Wn = Wc.copy(); Wn[0, 5] = w
        Wc, st, _, n = osci.osci_step(Wn, st, tau=4.0, window_end=(t == len(steps) - 1), reset_enabled=False)
    assert n == 0 and Wc[0, 5] == steps[-1]


def test_random_walk_invariants():
    r = np.random.default_rng(0)
    W = (r.standard_normal((32, 256)) * 0.02).astype(np.float32)
    st, _ = osci.osci_init(W)
    frozen = r.random(W.shape) < 0.3
    for t in range(1, 11):
        step = (r.standard_normal(W.shape) * 2e-4).astype(np.float32)
        step[frozen] = 0
        Wn = (W + step).astype(np.float32)
        Q_before, _ = osci.fwd_quant(Wn)
        W_out, st, Wq, n = osci.osci_step(Wn, st, tau=2.0, window_end=(t % 5 == 0), reset_enabled=True)
        changed = W_out != Wn
        # a reset sets the master exactly to its bin centre Q(w)
        np.testing.assert_array_equal(W_out[changed], Q_before[changed])
        np.testing.assert_array_equal(st.W_prev[changed], Q_before[changed])
        W = W_out
    np.testing.assert_array_equal(quant.dequantize(Wq), osci.fwd_quant(W)[0])


def test_topk_bruteforce_and_ties():
    r = np.random.default_rng(1)
    K = 64
    batches = [r.standard_normal((32, K)) * np.exp(r.standard_normal(K)) for _ in range(3)]
    s = calib.channel_scores(batches)
    got = calib.select_outliers(s, 0.1)
    assert len(got) == calib.n_outliers(K, 0.1) == 16
    ref = sorted(sorted(range(K), key=lambda c: (-s[c], c))[:16])
    assert list(got) == ref
    ties = np.array([1.0, 5.0, 5.0, 5.0] + [0.0] * 28)
    assert list(calib.select_outliers(ties, 0.5)) == list(range(16))
    assert calib.n_outliers(1024, 0.1) == 112 and calib.n_outliers(4096, 0.1) == 416

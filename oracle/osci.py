"""OsciReset state update (oracle; test infrastructure only).

OsciReset (TetraJet-v2 technical summary, section 2.B) tracks each weight's
trajectory and computes an oscillation risk: the distance travelled by the
quantized weight divided by the distance travelled by the master weight.  When
the learning rate is low and the risk exceeds a threshold, the master weight
is set to the centre of its current quantization bin.

Readings where the pages are silent:

* the quantized weight Q(w) is the forward quantizer's output (round-to-
  nearest, 1x16 groups along K, dequantized in fp32);
* "distance travelled" is the path length, the sum of |change| per optimizer
  step, accumulated over a tumbling window of steps;
* the risk test dQ / dM > tau is evaluated as dQ > tau * dM (fp32), so 0/0
  never resets and x/0 with x > 0 does;
* "centre of the current bin" is the bin's reconstruction point, i.e. Q(w);
* the learning-rate condition is a host-side switch (reset_enabled); the
  threshold tau and the window length are parameters.

One call per optimizer step, after the master update, in one of three modes:

* init:       Q = Q(W); W_prev = W; Q_prev = Q; dQ = dM = 0.
* accum:      Q = Q(W); dQ += |Q - Q_prev|; dM += |W - W_prev|;
              Q_prev = Q; W_prev = W.
* window_end: as accum, then where reset_enabled and dQ > tau * dM:
              W = Q and W_prev = Q; finally dQ = dM = 0.

The call also returns the forward codes of the final W for the next forward.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .quant import QTensor, dequantize, quantize


@dataclass
class OsciState:
    W_prev: np.ndarray
    Q_prev: np.ndarray
    dQ: np.ndarray
    dM: np.ndarray


def fwd_quant(W: np.ndarray) -> tuple[np.ndarray, QTensor]:
    Wq = quantize(np.asarray(W, dtype=np.float32), grouping="row", fmt="nvfp4", rounding="rtn")
    return dequantize(Wq), Wq


def osci_init(W: np.ndarray) -> tuple[OsciState, QTensor]:
    W = np.asarray(W, dtype=np.float32)
    Q, Wq = fwd_quant(W)
    z = np.zeros_like(W)
    return OsciState(W.copy(), Q, z.copy(), z.copy()), Wq


def osci_step(W: np.ndarray, st: OsciState, tau: float, window_end: bool, reset_enabled: bool):
    """Returns (W_new, state_new, Wq of W_new, number of resets)."""
    W = np.asarray(W, dtype=np.float32).copy()
    Q, _ = fwd_quant(W)
    dQ = (st.dQ + np.abs((Q - st.Q_prev).astype(np.float32))).astype(np.float32)
    dM = (st.dM + np.abs((W - st.W_prev).astype(np.float32))).astype(np.float32)
    Q_prev = Q.copy()
    W_prev = W.copy()
    n_reset = 0
    if window_end:
        if reset_enabled:
            hit = dQ > (np.float32(tau) * dM).astype(np.float32)
            n_reset = int(hit.sum())
            W = np.where(hit, Q, W).astype(np.float32)
            W_prev = np.where(hit, Q, W_prev).astype(np.float32)
        dQ = np.zeros_like(dQ)
        dM = np.zeros_like(dM)
    _, Wq = fwd_quant(W)
    return W, OsciState(W_prev, Q_prev, dQ, dM), Wq, n_reset

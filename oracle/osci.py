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

Oscillation diagnostics (optional, `diag` dict).  Section 1 of the technical
summary names the failure mode these measure: small master updates that make
the quantized weight flip back and forth between adjacent bins.

* flips: per accum / window_end call, the number of elements whose E2M1 code
  (the bin, with its sign) in the forward quantization of W differs from the
  code of the previous master W_prev, before any reset; +0 and -0 are one bin.
  Codes rather than dequantized values are compared because the per-128 scale
  moves with every update of a block's largest element, which changes Q(w) of
  the whole block without moving any element to another bin.  Summed by the
  caller over a window this is the window's flip count.
* risk_hist (window_end only): the window's risk dQ / dM of every element,
  taken before the reset decision and the zeroing, counted into RISK_BINS
  bins:  bin 0: dQ == 0;  bin 31: dQ > 0 and dM == 0;  otherwise with
  r = fl32(dQ / dM) and e = floor(log2 r) (the exponent of r), bin
  clamp(e + 16, 1, 30), so bin b in 2..29 holds r in [2^(b-16), 2^(b-15)) and
  bins 1 and 30 also take everything below 2^-14 and from 2^14 up.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .quant import QTensor, dequantize, quantize, unpack_nibbles


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


RISK_BINS = 32


def fwd_codes(W: np.ndarray) -> np.ndarray:
    """E2M1 code (sign bit 3, magnitude bits 0-2) of every element of the forward quantization of W."""
    return unpack_nibbles(fwd_quant(W)[1].codes)[:, : np.asarray(W).shape[1]]


def flip_count(W: np.ndarray, W_prev: np.ndarray) -> int:
    """Elements whose bin changed between the masters W_prev and W (+0 and -0 are one bin)."""
    c, cp = fwd_codes(W), fwd_codes(W_prev)
    same = (c == cp) | (((c & 7) == 0) & ((cp & 7) == 0))
    return int(np.count_nonzero(~same))


def risk_bin(dQ: np.ndarray, dM: np.ndarray) -> np.ndarray:
    """Per-element risk bin (see the module docstring) of the window's distances."""
    dQ = np.asarray(dQ, np.float32)
    dM = np.asarray(dM, np.float32)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        r = (dQ / dM).astype(np.float32)
    # exponent field of the non-negative fp32 quotient: floor(log2 r) for normal r
    e = ((r.view(np.uint32) >> np.uint32(23)) & np.uint32(0xFF)).astype(np.int64) - 127
    b = np.clip(e + 16, 1, 30)
    b = np.where(dM == 0, 31, b)
    return np.where(dQ == 0, 0, b).astype(np.int64)


def risk_histogram(dQ: np.ndarray, dM: np.ndarray) -> np.ndarray:
    return np.bincount(risk_bin(dQ, dM).ravel(), minlength=RISK_BINS).astype(np.int64)


def osci_step(W: np.ndarray, st: OsciState, tau: float, window_end: bool, reset_enabled: bool,
              diag: dict | None = None):
    """Returns (W_new, state_new, Wq of W_new, number of resets).  With diag, adds this
    call's flip count to diag["flips"] and, at a window end, the risk histogram to
    diag["risk_hist"] (both created when missing)."""
    W = np.asarray(W, dtype=np.float32).copy()
    Q, _ = fwd_quant(W)
    dQ = (st.dQ + np.abs((Q - st.Q_prev).astype(np.float32))).astype(np.float32)
    dM = (st.dM + np.abs((W - st.W_prev).astype(np.float32))).astype(np.float32)
    if diag is not None:
        diag["flips"] = diag.get("flips", 0) + flip_count(W, st.W_prev)
        if window_end:
            diag["risk_hist"] = diag.get("risk_hist", np.zeros(RISK_BINS, np.int64)) + risk_histogram(dQ, dM)
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

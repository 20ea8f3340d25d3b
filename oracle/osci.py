"""OsciReset state update (oracle; test infrastructure only).

OsciReset (TetraJet-v2 technical summary, section 2.B) tracks each weight's
trajectory and computes an oscillation risk: the distance travelled by the
quantized weight divided by the distance travelled by the master weight.  When
the learning rate is low and the risk exceeds a threshold, the master weight
is set to the centre of its current quantization bin.

Readings where the pages are silent:

* the quantized weight Q(w) is the forward quantizer's output (round-to-
  nearest, 1x16 groups along K, dequantized in fp32).  With a static
  OutControl plan (section 2.C) the forward quantizes the weights' outlier
  input channels to FP8 (E4M3, per-128 FP32 scale, round to nearest even) and
  the compacted remaining channels to NVFP4, so Q(w) follows the same split:
  an outlier-channel weight is reset to its FP8 reconstruction point, never to
  the coarser E2M1 grid;
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
  (the bin, with its sign; the E4M3 code for the FP8 channels of a plan) in the
  forward quantization of W differs from the code of the previous master
  W_prev, before any reset; +0 and -0 are one bin.
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


def fwd_quant(W: np.ndarray, plan=None):
    """Q(W) in fp32 and the forward codes: the NVFP4 QTensor, or (Wq, W8) with a plan (an object with
    sorted `rest` and `outliers` channel arrays): Wq NVFP4 over the compacted rest channels, W8 FP8
    (round to nearest even) over the outlier channels, Q scattered back to the channel order."""
    W = np.asarray(W, dtype=np.float32)
    if plan is None:
        Wq = quantize(W, grouping="row", fmt="nvfp4", rounding="rtn")
        return dequantize(Wq), Wq
    Wq = quantize(W[:, plan.rest], grouping="row", fmt="nvfp4", rounding="rtn")
    W8 = quantize(W[:, plan.outliers], grouping="row", fmt="fp8", rounding="rtn")
    Q = np.empty_like(W)
    Q[:, plan.rest] = dequantize(Wq)
    Q[:, plan.outliers] = dequantize(W8)
    return Q, (Wq, W8)


def osci_init(W: np.ndarray, plan=None):
    W = np.asarray(W, dtype=np.float32)
    Q, Wq = fwd_quant(W, plan)
    z = np.zeros_like(W)
    return OsciState(W.copy(), Q, z.copy(), z.copy()), Wq


RISK_BINS = 32


def fwd_codes(W: np.ndarray, plan=None):
    """E2M1 code (sign bit 3, magnitude bits 0-2) of every element of the forward quantization of W;
    with a plan, (E2M1 codes of the rest channels, E4M3 codes of the outlier channels)."""
    W = np.asarray(W)
    if plan is None:
        return unpack_nibbles(fwd_quant(W)[1].codes)[:, : W.shape[1]]
    Wq, W8 = fwd_quant(W, plan)[1]
    return unpack_nibbles(Wq.codes)[:, : len(plan.rest)], W8.codes[:, : len(plan.outliers)]


def flip_count(W: np.ndarray, W_prev: np.ndarray, plan=None) -> int:
    """Elements whose bin changed between the masters W_prev and W (+0 and -0 are one bin)."""
    if plan is None:
        c, cp = fwd_codes(W), fwd_codes(W_prev)
        same = (c == cp) | (((c & 7) == 0) & ((cp & 7) == 0))
        return int(np.count_nonzero(~same))
    (c4, c8), (p4, p8) = fwd_codes(W, plan), fwd_codes(W_prev, plan)
    same4 = (c4 == p4) | (((c4 & 7) == 0) & ((p4 & 7) == 0))
    same8 = (c8 == p8) | (((c8 & 0x7F) == 0) & ((p8 & 0x7F) == 0))
    return int(np.count_nonzero(~same4) + np.count_nonzero(~same8))


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
              diag: dict | None = None, plan=None):
    """Returns (W_new, state_new, forward codes of W_new, number of resets); the codes are those
    of fwd_quant (a QTensor, or (Wq, W8) with a plan).  With diag, adds this call's flip count
    to diag["flips"] and, at a window end, the risk histogram to diag["risk_hist"] (both
    created when missing)."""
    W = np.asarray(W, dtype=np.float32).copy()
    Q, _ = fwd_quant(W, plan)
    dQ = (st.dQ + np.abs((Q - st.Q_prev).astype(np.float32))).astype(np.float32)
    dM = (st.dM + np.abs((W - st.W_prev).astype(np.float32))).astype(np.float32)
    if diag is not None:
        diag["flips"] = diag.get("flips", 0) + flip_count(W, st.W_prev, plan)
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
    _, Wq = fwd_quant(W, plan)
    return W, OsciState(W_prev, Q_prev, dQ, dM), Wq, n_reset

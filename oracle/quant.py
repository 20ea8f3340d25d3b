"""Double-block NVFP4 and per-block FP8 quantizers (oracle; test infrastructure only).

Double-block structure (TetraJet-v2 technical summary, section 2.A): an
outer block of 128 consecutive elements along the grouping dimension carries
an FP32 scale; each of its inner blocks of 16 elements carries an 8-bit
(E4M3) scale; elements are E2M1.  No amax over the whole tensor is taken.
Weights use 1x16 groups; the transposed operands of the backward products are
re-grouped along the other dimension (16x1 groups, stored transposed).

Readings where the pages are silent (all fp32, one IEEE operation at a time):

* outer scale: a_o = max |y| over the outer block (the last block of a row
  may be shorter, a multiple of 16).  If a_o < 2^-100 the block is "empty":
  S = 0, every inner scale 0, every code carries only the input's sign.
  Otherwise S = a_o / 2688, where 2688 = 6 * 448 maps the block maximum onto
  the largest E2M1 value times the largest E4M3 value.
* inner scale: a_j = max |y| over the 16 elements; a_j = 0 gives s = 0;
  otherwise r = a_j / (6 * S) and s = the smallest E4M3FN value >= min(r, 448)
  (rounding *up* keeps every scaled element within +-6, so no element is
  clipped, which stochastic rounding needs to stay unbiased).
* element: d = s * S, inv = 1 / d, v = clamp(y * inv, -6, 6), then the
  round-to-nearest (forward) or stochastic (backward) E2M1 rule.
* dequantized value: (q * s) * S, the product q * s being exact.

NVFP6 (the FP6 x FP4 variant the pages name as future work, section 5): the
same double block with E2M3 elements (largest 7.5): S = a_o / 3360 (7.5 * 448),
s = the smallest E4M3FN value >= min(a_j / (7.5 * S), 448), v = clamp(y * inv,
-7.5, 7.5), then the E2M3 round-to-nearest or stochastic rule; each element
is stored as the E4M3FN byte of its E2M3 value (one byte per element).

FP8 outlier channels (section 2.C, "e.g. FP8"): OCP E4M3FN elements with one
FP32 scale per 128 elements along the grouping dimension: S8 = a_o / 448,
v = clamp(y * (1 / S8), -448, 448), round-to-nearest-even (forward) or the
same stochastic rule on the E4M3 grid (backward); same empty-block rule.

Storage (oracle side): codes uint8 [rows, L/2] (NVFP4, element 2i in the low
nibble of byte i) or [rows, L] (FP8); s16 uint8 [rows, L/16]; s128 float32
[rows, ceil(L/128)].  The HIP library pads rows to whole outer blocks; the
tests compare the unpadded region.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import formats, philox, rht

TINY = np.float32(2.0 ** -100)
NVFP4_OUTER_DIV = np.float32(2688.0)  # 6 * 448
NVFP6_OUTER_DIV = np.float32(3360.0)  # 7.5 * 448
FP8_OUTER_DIV = np.float32(448.0)


@dataclass
class QTensor:
    fmt: str  # "nvfp4" or "fp8"
    codes: np.ndarray
    s128: np.ndarray
    s16: np.ndarray | None
    rows: int
    L: int


def _outer_amax(a: np.ndarray, L: int):
    rows = a.shape[0]
    nb = -(-L // 128)
    pad = np.zeros((rows, nb * 128), dtype=np.float32)
    pad[:, :L] = a
    return pad.reshape(rows, nb, 128).max(axis=-1), nb


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] & 0xF) | ((c[:, 1::2] & 0xF) << 4)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def nvfp4_quantize_rows(y: np.ndarray, rounding: str = "rtn", u16=None) -> QTensor:
    """Double-block NVFP4 quantization of fp32 y [rows, L] along its last axis."""
    return _double_block_rows(y, rounding, u16, fp6=False)


def nvfp6_quantize_rows(y: np.ndarray, rounding: str = "rtn", u16=None) -> QTensor:
    """Double-block NVFP6 (E2M3 elements) quantization of fp32 y [rows, L] along its last axis."""
    return _double_block_rows(y, rounding, u16, fp6=True)


def _double_block_rows(y: np.ndarray, rounding: str, u16, fp6: bool) -> QTensor:
    y = np.asarray(y, dtype=np.float32)
    rows, L = y.shape
    assert L % 16 == 0 and L > 0
    emax = np.float32(7.5 if fp6 else 6.0)
    a = np.abs(y)
    a_o, nb = _outer_amax(a, L)
    empty_o = a_o < TINY
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        S = np.where(empty_o, np.float32(0), a_o / (NVFP6_OUTER_DIV if fp6 else NVFP4_OUTER_DIV)).astype(np.float32)
        a_j = a.reshape(rows, L // 16, 16).max(axis=-1)
        S_j = S[:, np.arange(L // 16) // 8]
        six_S = (emax * S_j).astype(np.float32)
        r = np.where(six_S > 0, a_j / np.where(six_S > 0, six_S, np.float32(1)), np.float32(0)).astype(np.float32)
        r = np.minimum(r, np.float32(formats.E4M3_MAX))
        empty_j = (a_j == 0) | (S_j == 0)
        s_code = np.where(empty_j, 0, formats.e4m3_round_up(np.where(empty_j, np.float32(1), r))).astype(np.uint8)
        s_val = formats.e4m3_decode(s_code).astype(np.float32)
        d = (s_val * S_j).astype(np.float32)
        inv = np.where(d > 0, np.float32(1.0) / np.where(d > 0, d, np.float32(1)), np.float32(0)).astype(np.float32)
        inv_e = np.repeat(inv, 16, axis=1)
        v = (y * inv_e).astype(np.float32)
    v = np.minimum(np.maximum(v, -emax), emax)
    empty_e = np.repeat(empty_j, 16, axis=1)
    v = np.where(empty_e, np.copysign(np.float32(0), y), v).astype(np.float32)
    if rounding not in ("rtn", "sr"):
        raise ValueError(rounding)
    if fp6:
        q = formats.e2m3_rtn(v) if rounding == "rtn" else formats.e2m3_sr(v, u16)
        return QTensor("nvfp6", formats.e2m3_to_e4m3(q), S, s_code, rows, L)
    q = formats.e2m1_rtn(v) if rounding == "rtn" else formats.e2m1_sr(v, u16)
    return QTensor("nvfp4", pack_nibbles(q), S, s_code, rows, L)


def fp8_quantize_rows(y: np.ndarray, rounding: str = "rtn", u16=None) -> QTensor:
    """Per-128-block E4M3FN quantization of fp32 y [rows, L] along its last axis."""
    y = np.asarray(y, dtype=np.float32)
    rows, L = y.shape
    assert L % 16 == 0 and L > 0
    a_o, nb = _outer_amax(np.abs(y), L)
    empty_o = a_o < TINY
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        S = np.where(empty_o, np.float32(0), a_o / FP8_OUTER_DIV).astype(np.float32)
        inv = np.where(S > 0, np.float32(1.0) / np.where(S > 0, S, np.float32(1)), np.float32(0)).astype(np.float32)
        inv_e = np.repeat(inv, 128, axis=1)[:, :L]
        v = (y * inv_e).astype(np.float32)
    v = np.minimum(np.maximum(v, np.float32(-formats.E4M3_MAX)), np.float32(formats.E4M3_MAX))
    empty_e = np.repeat(empty_o, 128, axis=1)[:, :L]
    v = np.where(empty_e, np.copysign(np.float32(0), y), v).astype(np.float32)
    if rounding == "rtn":
        q = formats.e4m3_rne(v)
    elif rounding == "sr":
        q = formats.e4m3_sr(v, u16)
    else:
        raise ValueError(rounding)
    return QTensor("fp8", q, S, None, rows, L)


def dequantize(q: QTensor) -> np.ndarray:
    """fp32 dequantized values: (q * s) * S for NVFP4, e * S8 for FP8."""
    rows, L = q.rows, q.L
    S_e = np.repeat(q.s128, 128, axis=1)[:, :L].astype(np.float32)
    if q.fmt in ("nvfp4", "nvfp6"):
        qv = (formats.e2m1_decode(unpack_nibbles(q.codes)) if q.fmt == "nvfp4" else
              formats.e4m3_decode(q.codes)).astype(np.float32)
        s_e = np.repeat(formats.e4m3_decode(q.s16).astype(np.float32), 16, axis=1)
        return ((qv * s_e).astype(np.float32) * S_e).astype(np.float32)
    ev = formats.e4m3_decode(q.codes).astype(np.float32)
    return (ev * S_e).astype(np.float32)


def dequantize_f64(q: QTensor) -> np.ndarray:
    """Exact fp64 value q * s * S (the operand value of the reference products)."""
    L = q.L
    S_e = np.repeat(q.s128.astype(np.float64), 128, axis=1)[:, :L]
    if q.fmt in ("nvfp4", "nvfp6"):
        qv = formats.e2m1_decode(unpack_nibbles(q.codes)) if q.fmt == "nvfp4" else formats.e4m3_decode(q.codes)
        s_e = np.repeat(formats.e4m3_decode(q.s16), 16, axis=1)
        return qv * s_e * S_e
    return formats.e4m3_decode(q.codes) * S_e


def quantize(x: np.ndarray, *, grouping: str = "row", fmt: str = "nvfp4", rounding: str = "rtn",
             rht_mask: int | None = None, seed: int = 0, offset: int = 0) -> QTensor:
    """Quantize fp32 x [R, C].

    grouping "row": groups run along C, the result is [R, C].
    grouping "col": groups run along R (16x1), the result is stored transposed, [C, R].
    rht_mask: if given, the 16-wide Hadamard transform with that sign mask is
    applied along the grouping dimension before quantizing.
    Stochastic draws are indexed by the element's row-major position in the
    (grouped, possibly transposed) output.
    """
    x = np.asarray(x, dtype=np.float32)
    R, C = x.shape
    if grouping == "row":
        xg = x
    elif grouping == "col":
        xg = np.ascontiguousarray(x.T)
    else:
        raise ValueError(grouping)
    y = rht.rht_along_last(xg, rht_mask) if rht_mask is not None else xg
    u16 = philox.sr_draws_for_shape(y.shape, seed, offset) if rounding == "sr" else None
    if fmt == "nvfp4":
        return nvfp4_quantize_rows(y, rounding, u16)
    if fmt == "nvfp6":
        return nvfp6_quantize_rows(y, rounding, u16)
    if fmt == "fp8":
        return fp8_quantize_rows(y, rounding, u16)
    raise ValueError(fmt)

"""Number formats of the double-block NVFP4 scheme (oracle; test infrastructure only).

NVFP4 elements are E2M1 with an 8-bit scale per 16 elements (TetraJet-v2
technical summary, section 2.A).  The element grid {0, 0.5, 1, 1.5, 2, 3, 4, 6}
and the E4M3FN scale type are the standard OCP definitions of those formats;
the pages name the formats but do not spell out their bit layouts, so the
layouts below are the OCP ones:

* E2M1 code (4 bits): bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa.
  Exponent 0 is subnormal (value = m * 0.5).
* E4M3FN (8 bits): bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0
  mantissa; exponent 0 is subnormal (m * 2^-9); 0x7F / 0xFF are NaN; no
  infinities; largest finite 448.

* E2M3 (6 bits, the FP6 operand of the FP6 x FP4 variant the pages name as
  future work): bit 5 sign, bits 4..3 exponent (bias 1), bits 2..0 mantissa;
  exponent 0 is subnormal (value = m * 0.125); largest value 7.5.  Every
  E2M3 value is an E4M3FN value, which is how the library stores them.

Element rounding rules (readings where the pages are silent):
* round-to-nearest (forward pass): nearest grid value, a tie goes to the code
  whose mantissa bit is 0 (IEEE-style ties-to-even); the sign of the input is
  kept, so -0 encodes as code 8.
* stochastic rounding (backward pass, E[round(x)] = x per section 2.A): with
  lo <= |v| < hi the neighbouring grid values and t = (|v| - lo) / (hi - lo)
  * 65536 (exact in fp32), round up iff a 16-bit uniform draw u satisfies
  u + floor(t) >= 65536, i.e. the fraction plus u / 65536 reaches the next
  grid value.  P(up) = floor(t) / 65536, within 2^-16 of the exact fraction.
  The pages fix only unbiasedness; this form of the rule is what gfx950's
  stochastic conversion instructions compute when the draw occupies the top
  16 bits of their random operand.
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# E2M1
# ---------------------------------------------------------------------------


def e2m1_decode(code) -> np.ndarray:
    """Value (fp64) of 4-bit E2M1 codes, from the bit fields."""
    c = np.asarray(code).astype(np.int64) & 0xF
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, m * 0.5, np.ldexp(1.0 + 0.5 * m, np.maximum(e - 1, 0)))
    return np.where(s == 1, -mag, mag)


#: magnitudes of codes 0..7 in code order (ascending)
E2M1_MAG = e2m1_decode(np.arange(8))


def _e2m1_floor_index(a64: np.ndarray) -> np.ndarray:
    """Index of the largest grid magnitude <= a (a >= 0)."""
    return np.clip(np.searchsorted(E2M1_MAG, a64, side="right") - 1, 0, 7)


def e2m1_rtn(v) -> np.ndarray:
    """Round fp32 values (|v| <= 6) to E2M1 codes, nearest with ties to even mantissa."""
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v).astype(np.float64)
    lo = _e2m1_floor_index(a)
    hi = np.minimum(lo + 1, 7)
    d_lo = a - E2M1_MAG[lo]
    d_hi = E2M1_MAG[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi != lo) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo).astype(np.uint8)
    return idx | (np.signbit(v).astype(np.uint8) << 3)


def e2m1_sr(v, u16) -> np.ndarray:
    """Stochastically round fp32 values (|v| <= 6) to E2M1 codes with 16-bit draws u16."""
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v)
    lo = _e2m1_floor_index(a.astype(np.float64))
    hi = np.minimum(lo + 1, 7)
    lo_v = E2M1_MAG[lo].astype(np.float32)
    gap = (E2M1_MAG[hi] - E2M1_MAG[lo]).astype(np.float32)
    with np.errstate(invalid="ignore", divide="ignore"):
        p = np.where(gap > 0, (a - lo_v) / np.where(gap > 0, gap, np.float32(1)), np.float32(0)).astype(np.float32)
    t = (p * np.float32(65536.0)).astype(np.float32)
    up = np.asarray(u16, dtype=np.uint16).astype(np.int64) + np.floor(t).astype(np.int64) >= 65536
    idx = np.where(up, hi, lo).astype(np.uint8)
    return idx | (np.signbit(v).astype(np.uint8) << 3)


# ---------------------------------------------------------------------------
# E4M3FN
# ---------------------------------------------------------------------------


def e4m3_decode(code) -> np.ndarray:
    """Value (fp64) of E4M3FN bytes, from the bit fields (NaN for 0x7F/0xFF)."""
    c = np.asarray(code).astype(np.int64) & 0xFF
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, np.ldexp(1.0 + m / 8.0, np.maximum(e - 7, -6)))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


#: values of the non-negative finite codes 0x00..0x7E, ascending in code order
E4M3_POS = e4m3_decode(np.arange(0x7F))
E4M3_MAX = 448.0


def e4m3_round_up(r) -> np.ndarray:
    """Code of the smallest E4M3FN value >= r, for fp32 0 < r <= 448."""
    r = np.asarray(r, dtype=np.float32).astype(np.float64)
    return np.searchsorted(E4M3_POS, r, side="left").astype(np.uint8)


def e4m3_rne(v) -> np.ndarray:
    """E4M3FN code of fp32 v (|v| <= 448): nearest, ties to even code; sign kept."""
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v).astype(np.float64)
    lo = np.clip(np.searchsorted(E4M3_POS, a, side="right") - 1, 0, 0x7E)
    hi = np.minimum(lo + 1, 0x7E)
    d_lo = a - E4M3_POS[lo]
    d_hi = E4M3_POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi != lo) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo).astype(np.uint8)
    return idx | (np.signbit(v).astype(np.uint8) << 7)


def e4m3_sr(v, u16) -> np.ndarray:
    """Stochastic rounding of fp32 v (|v| <= 448) onto the E4M3FN grid (same rule as E2M1)."""
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v)
    lo = np.clip(np.searchsorted(E4M3_POS, a.astype(np.float64), side="right") - 1, 0, 0x7E)
    hi = np.minimum(lo + 1, 0x7E)
    lo_v = E4M3_POS[lo].astype(np.float32)
    gap = (E4M3_POS[hi] - E4M3_POS[lo]).astype(np.float32)
    with np.errstate(invalid="ignore", divide="ignore"):
        p = np.where(gap > 0, (a - lo_v) / np.where(gap > 0, gap, np.float32(1)), np.float32(0)).astype(np.float32)
    t = (p * np.float32(65536.0)).astype(np.float32)
    up = np.asarray(u16, dtype=np.uint16).astype(np.int64) + np.floor(t).astype(np.int64) >= 65536
    idx = np.where(up, hi, lo).astype(np.uint8)
    return idx | (np.signbit(v).astype(np.uint8) << 7)


# ---------------------------------------------------------------------------
# E2M3 (FP6)
# ---------------------------------------------------------------------------


def e2m3_decode(code) -> np.ndarray:
    """Value (fp64) of 6-bit E2M3 codes, from the bit fields."""
    c = np.asarray(code).astype(np.int64) & 0x3F
    s = (c >> 5) & 1
    e = (c >> 3) & 3
    m = c & 7
    mag = np.where(e == 0, m * 0.125, np.ldexp(1.0 + m / 8.0, np.maximum(e - 1, 0)))
    return np.where(s == 1, -mag, mag)


#: magnitudes of codes 0..31 in code order (ascending): 0, 0.125, ..., 7.5
E2M3_MAG = e2m3_decode(np.arange(32))


def _e2m3_floor_index(a64: np.ndarray) -> np.ndarray:
    return np.clip(np.searchsorted(E2M3_MAG, a64, side="right") - 1, 0, 31)


def e2m3_rtn(v) -> np.ndarray:
    """Round fp32 values (|v| <= 7.5) to E2M3 codes, nearest with ties to even mantissa; sign kept."""
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v).astype(np.float64)
    lo = _e2m3_floor_index(a)
    hi = np.minimum(lo + 1, 31)
    d_lo = a - E2M3_MAG[lo]
    d_hi = E2M3_MAG[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi != lo) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo).astype(np.uint8)
    return idx | (np.signbit(v).astype(np.uint8) << 5)


def e2m3_sr(v, u16) -> np.ndarray:
    """Stochastic rounding of fp32 values (|v| <= 7.5) onto the E2M3 grid (same rule as E2M1)."""
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v)
    lo = _e2m3_floor_index(a.astype(np.float64))
    hi = np.minimum(lo + 1, 31)
    lo_v = E2M3_MAG[lo].astype(np.float32)
    gap = (E2M3_MAG[hi] - E2M3_MAG[lo]).astype(np.float32)
    with np.errstate(invalid="ignore", divide="ignore"):
        p = np.where(gap > 0, (a - lo_v) / np.where(gap > 0, gap, np.float32(1)), np.float32(0)).astype(np.float32)
    t = (p * np.float32(65536.0)).astype(np.float32)
    up = np.asarray(u16, dtype=np.uint16).astype(np.int64) + np.floor(t).astype(np.int64) >= 65536
    idx = np.where(up, hi, lo).astype(np.uint8)
    return idx | (np.signbit(v).astype(np.uint8) << 5)


def e2m3_to_e4m3(code6) -> np.ndarray:
    """The E4M3FN byte of the same value as each E2M3 code (the library's storage of FP6 elements)."""
    c = np.asarray(code6).astype(np.int64) & 0x3F
    mag = e2m3_decode(c & 0x1F)
    idx = np.searchsorted(E4M3_POS, mag)
    assert np.all(E4M3_POS[idx] == mag)
    return (idx | ((c >> 5) << 7)).astype(np.uint8)

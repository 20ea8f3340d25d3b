"""Counter-based random numbers for stochastic rounding (oracle; test infrastructure only).

The backward quantizers round stochastically (TetraJet-v2 technical summary,
section 2.A).  The pages do not fix a generator; the reading taken here is
the standard Philox4x32 with 10 rounds (Salmon, Moraes, Dror, Shaw,
"Parallel random numbers: as easy as 1, 2, 3", SC'11):

* one round maps (c0, c1, c2, c3) with key (k0, k1) to
  (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1, lo(M0*c0)),
  M0 = 0xD2511F53, M1 = 0xCD9E8D57;
* the key is bumped by (0x9E3779B9, 0xBB67AE85) between rounds.

Per-element draw (reading): the element with row-major index e in the
quantizer's *output* array (the grouped layout: for a transposed 16x1
quantization, output row = input column) uses block b = e >> 3 with counter
(lo32 b, hi32 b, lo32 offset, hi32 offset) and key (lo32 seed, hi32 seed);
its 16-bit draw is half (e & 1) (0 = low half) of output word (e >> 1) & 3.
Every 16-element group therefore consumes exactly two whole Philox blocks.

RHT signs for one GEMM pair: the low 16 bits of word 0 of the block with
counter (0xFFFFFFFF, 0xFFFFFFFF, lo32 offset, hi32 offset); bit j set means
position j of every 16-chunk is negated.

Two implementations (pure-Python integers and vectorised numpy) are kept and
must agree; the tests also compare against rocrand's Philox4x32-10.
"""
from __future__ import annotations

import numpy as np

M0, M1 = 0xD2511F53, 0xCD9E8D57
W0, W1 = 0x9E3779B9, 0xBB67AE85
MASK32 = 0xFFFFFFFF
ROUNDS = 10


def philox4x32_10_scalar(ctr, key):
    """Pure-Python Philox4x32-10 of one counter block -> tuple of 4 ints."""
    c0, c1, c2, c3 = (int(c) & MASK32 for c in ctr)
    k0, k1 = (int(k) & MASK32 for k in key)
    for r in range(ROUNDS):
        if r:
            k0 = (k0 + W0) & MASK32
            k1 = (k1 + W1) & MASK32
        p0 = M0 * c0
        p1 = M1 * c2
        c0, c1, c2, c3 = ((p1 >> 32) ^ c1 ^ k0, p1 & MASK32, (p0 >> 32) ^ c3 ^ k1, p0 & MASK32)
    return c0, c1, c2, c3


def philox4x32_10(c0, c1, c2, c3, k0: int, k1: int):
    """Vectorised Philox4x32-10: arrays of uint32 counters -> 4 uint32 arrays."""
    c = [np.asarray(x, dtype=np.uint64) & np.uint64(MASK32) for x in (c0, c1, c2, c3)]
    c0, c1, c2, c3 = np.broadcast_arrays(*c)
    c0, c1, c2, c3 = (x.copy() for x in (c0, c1, c2, c3))
    m32 = np.uint64(MASK32)
    s32 = np.uint64(32)
    for r in range(ROUNDS):
        kk0 = np.uint64((k0 + r * W0) & MASK32)
        kk1 = np.uint64((k1 + r * W1) & MASK32)
        p0 = c0 * np.uint64(M0)  # < 2^64: exact in uint64
        p1 = c2 * np.uint64(M1)
        c0, c1, c2, c3 = ((p1 >> s32) ^ c1 ^ kk0, p1 & m32, (p0 >> s32) ^ c3 ^ kk1, p0 & m32)
    return tuple(x.astype(np.uint32) for x in (c0, c1, c2, c3))


def sr_draws_u16(e, seed: int, offset: int) -> np.ndarray:
    """16-bit uniform draw for each element index e (int array) of one quantizer call."""
    e = np.asarray(e, dtype=np.uint64)
    b = e >> np.uint64(3)
    words = philox4x32_10(b & np.uint64(MASK32), b >> np.uint64(32),
                          np.uint64(offset & MASK32), np.uint64((offset >> 32) & MASK32),
                          seed & MASK32, (seed >> 32) & MASK32)
    w = np.stack(words, axis=0)  # (4, ...)
    sel = ((e >> np.uint64(1)) & np.uint64(3)).astype(np.int64)
    word = np.take_along_axis(w, sel[None, ...], axis=0)[0]
    half = (e & np.uint64(1)).astype(np.uint32)
    return ((word >> (half * np.uint32(16))) & np.uint32(0xFFFF)).astype(np.uint16)


def sr_draws_for_shape(shape, seed: int, offset: int) -> np.ndarray:
    """Draws for every element of a row-major array of `shape`, indexed by position."""
    n = int(np.prod(shape))
    return sr_draws_u16(np.arange(n, dtype=np.uint64), seed, offset).reshape(shape)


def rht_signs(seed: int, offset: int) -> int:
    """16-bit sign mask of the random Hadamard transform for one GEMM pair."""
    w = philox4x32_10_scalar((MASK32, MASK32, offset & MASK32, (offset >> 32) & MASK32),
                             (seed & MASK32, (seed >> 32) & MASK32))
    return w[0] & 0xFFFF

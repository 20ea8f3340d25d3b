"""Seeded synthetic inputs shared by the tests, the bench and the oracle.

This module only draws random numbers and rounds them to the storage types
(bf16 with round-to-nearest-even, fp32).  It holds none of the quantization,
transform, GEMM or OsciReset arithmetic; the CPU oracle and the HIP library
each implement that on their own and both read the bytes produced here.

Workload shapes follow the OLMo-2-style linear layers the TetraJet-v2 pages
evaluate on (70M and 370M models; technical summary, section 4): the
synthetic tensors stand in for the pretraining data, which is not available.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# ---------------------------------------------------------------------------
# storage-type helpers (bit-level, no method arithmetic)
# ---------------------------------------------------------------------------


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bf16 (round-to-nearest-even); returns uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    out = np.empty(b.shape, np.uint16)
    flat_b, flat_o = b.reshape(-1), out.reshape(-1)
    step = 1 << 22  # chunks keep the temporaries small; finite inputs never overflow 32 bits
    for i in range(0, flat_b.size, step):
        c = flat_b[i:i + step]
        flat_o[i:i + step] = (c + (np.uint32(0x7FFF) + ((c >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)
    return out


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """Widen bf16 bits (uint16) to fp32 exactly."""
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------------------
# generators
# ---------------------------------------------------------------------------


def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def normal_bf16(shape, std: float, seed: int) -> np.ndarray:
    """bf16 bits of N(0, std^2) samples (std is a standard deviation)."""
    z = rng(seed).standard_normal(size=shape, dtype=np.float32) * np.float32(std)
    return f32_to_bf16_bits(z)


def normal_f32(shape, std: float, seed: int) -> np.ndarray:
    return rng(seed).standard_normal(size=shape, dtype=np.float32) * np.float32(std)


def outlier_columns(n_cols: int, frac: float, seed: int) -> np.ndarray:
    """round(frac * n_cols) distinct random column indices (sorted)."""
    n = int(round(frac * n_cols))
    return np.sort(rng(seed).choice(n_cols, size=n, replace=False)).astype(np.int64)


def acts_with_outliers_bf16(shape, std: float, frac: float, gain: float, seed: int) -> np.ndarray:
    """N(0, std^2) activations with round(frac*K) channels scaled by `gain` (bf16 bits)."""
    z = rng(seed).standard_normal(size=shape, dtype=np.float32) * np.float32(std)
    cols = outlier_columns(shape[-1], frac, seed + 7919)
    z[..., cols] *= np.float32(gain)
    return f32_to_bf16_bits(z)


def lognormal_channel_gains(n_cols: int, sigma: float, seed: int) -> np.ndarray:
    """Fixed per-channel gains g_c = exp(sigma * zeta_c), zeta_c ~ N(0,1) (fp32)."""
    return np.exp(np.float32(sigma) * rng(seed).standard_normal(n_cols, dtype=np.float32)).astype(np.float32)


def heavy_tailed_acts_bf16(n_rows: int, gains: np.ndarray, seed: int) -> np.ndarray:
    """X[t, c] = z * g_c with z ~ N(0,1): heavy-tailed channel norms (bf16 bits)."""
    z = rng(seed).standard_normal(size=(n_rows, gains.shape[0]), dtype=np.float32)
    return f32_to_bf16_bits(z * gains[None, :])


# ---------------------------------------------------------------------------
# workload descriptions
# ---------------------------------------------------------------------------


@dataclass(frozen=True)
class LinearShape:
    name: str
    K: int  # in-features
    N: int  # out-features


@dataclass
class Workload:
    name: str
    M: int
    layers: int
    linears: list = field(default_factory=list)

    def gemm_flops_per_step(self) -> float:
        """2*M*N*K for fwd, dX and dW of every linear (algorithmic flops only)."""
        return float(sum(6 * self.M * l.N * l.K for l in self.linears) * self.layers)


def olmo_linears(d_model: int, ffn: int) -> list:
    return [
        LinearShape("qkv", d_model, 3 * d_model),
        LinearShape("o", d_model, d_model),
        LinearShape("gate", d_model, ffn),
        LinearShape("up", d_model, ffn),
        LinearShape("down", ffn, d_model),
    ]


SINGLE_LINEAR = Workload("single-linear-256x512x512", M=256, layers=1,
                         linears=[LinearShape("single", 512, 512)])
QUANT_SWEEP_SHAPE = (8192, 4096)
OLMO70M = Workload("olmo2-70M-style-linears-M16384", M=16384, layers=8, linears=olmo_linears(512, 2048))
OLMO370M = Workload("olmo2-370M-style-linears-M16384", M=16384, layers=16, linears=olmo_linears(1024, 4096))


def outlier_count(K: int, p: float) -> int:
    """Number of statically retained channels: top p of K, rounded up to a multiple of 16."""
    return int(math.ceil(p * K / 16.0)) * 16


# Seeds are fixed per tensor role so every consumer regenerates identical bytes.
SEED_X, SEED_W, SEED_DY, SEED_GAIN, SEED_CALIB = 1001, 2002, 3003, 4004, 5005

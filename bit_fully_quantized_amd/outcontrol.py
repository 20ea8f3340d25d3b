"""OutControl calibration policy (host side of a one-off step, not the hot path).

TetraJet-v2 technical summary, section 2.C: outlier channels are structurally
consistent, so the top p% input channels are picked once from a short
calibration window and kept in FP8 afterwards.  The per-channel sums of
squares are accumulated on the GPU by tj2_channel_sumsq; the ranking (fp64,
ties to the lower channel index) and the count (ceil(p*K/16)*16, so the NVFP4
remainder stays a whole number of 16-element groups) are applied here.
"""
from __future__ import annotations

import math

import torch

from . import OutlierPlan, channel_sumsq


def n_outliers(K: int, p: float) -> int:
    return int(math.ceil(p * K / 16.0)) * 16


def calibrate(batches, p: float = 0.10) -> OutlierPlan:
    """batches: iterable of bf16 device tensors [M_b, K] (the layer's inputs)."""
    total = None
    for X in batches:
        acc = torch.zeros(X.shape[1], dtype=torch.float32, device=X.device)
        channel_sumsq(X, acc)
        total = acc.double() if total is None else total + acc.double()
    K = total.numel()
    order = torch.sort(total, descending=True, stable=True).indices
    chosen = torch.sort(order[: n_outliers(K, p)]).values
    return OutlierPlan.from_indices(K, chosen.cpu().tolist(), device=total.device)

"""OutControl calibration (a one-off step before training, not the hot path).

TetraJet-v2 technical summary, section 2.C: outlier channels are structurally
consistent, so the top p% input channels are picked once from a short
calibration window and kept in FP8 afterwards.  Both steps run in the library:
tj2_channel_sumsq accumulates the per-channel sums of squares on the GPU (fp64,
fixed order) and tj2_select_outliers ranks them (ties to the lower channel, a
count of ceil(p*K/16)*16 so the NVFP4 remainder stays whole 16-element groups).
"""
from __future__ import annotations

import torch

from . import OutlierPlan, channel_sumsq, n_outliers, select_outliers  # noqa: F401


def calibrate(batches, p: float = 0.10) -> OutlierPlan:
    """batches: iterable of bf16 device tensors [M_b, K] (the layer's inputs)."""
    acc = None
    for X in batches:
        if acc is None:
            acc = torch.zeros(X.shape[1], dtype=torch.float64, device=X.device)
        channel_sumsq(X, acc)
    return select_outliers(acc, p, device=acc.device)

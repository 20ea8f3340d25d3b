"""OutControl calibration (oracle; test infrastructure only).

Outlier channels are structurally consistent, so the top p% input channels
are chosen once during a short calibration window and kept in FP8 afterwards
(TetraJet-v2 technical summary, section 2.C; p = 10% is the pages' example).

Readings: the channel score is the sum of squares of the channel over all
calibration tokens (fp64); the number kept is ceil(p * K / 16) * 16 so the
NVFP4 remainder stays a whole number of 16-element groups; ties go to the lower
channel index; the result is sorted ascending.
"""
from __future__ import annotations

import math

import numpy as np


def channel_scores(batches) -> np.ndarray:
    acc = None
    for X in batches:
        s = np.sum(np.asarray(X, dtype=np.float64) ** 2, axis=0)
        acc = s if acc is None else acc + s
    return acc


def n_outliers(K: int, p: float) -> int:
    return int(math.ceil(p * K / 16.0)) * 16


def select_outliers(scores: np.ndarray, p: float) -> np.ndarray:
    K = scores.shape[0]
    n = n_outliers(K, p)
    order = np.lexsort((np.arange(K), -scores))  # descending score, then ascending index
    return np.sort(order[:n]).astype(np.int64)

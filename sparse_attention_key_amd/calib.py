"""Host-side calibration statistics (run once per (layer, KV head), off the
decode path).

The water-filling weight needs each stored coordinate's key variance, measured
once on calibration keys; the rotated storage needs the eigenbasis of the
calibration key covariance ordered by decreasing variance (yeyulingfeng.com
write-up of Fathom, reverse water-filling section and basis-choice section).
Variances are centred population variances accumulated in float64 and
rounded once to float32.
"""
from __future__ import annotations

import numpy as np


def channel_variance(sample: np.ndarray) -> np.ndarray:
    """sample [m][D] -> sigma^2 [D] float32."""
    x = np.asarray(sample, np.float64)
    return x.var(axis=0).astype(np.float32)


def rotation(sample: np.ndarray):
    """sample [m][D] -> (U [D][D] float32 with eigenvector columns ordered by
    descending eigenvalue, lam [D] float32 variances of the rotated
    coordinates, clamped at 0)."""
    x = np.asarray(sample, np.float64)
    xc = x - x.mean(axis=0, keepdims=True)
    cov = (xc.T @ xc) / x.shape[0]
    lam, vec = np.linalg.eigh(cov)
    order = np.argsort(lam)[::-1]
    return np.ascontiguousarray(vec[:, order], np.float32), np.maximum(lam[order], 0.0).astype(np.float32)

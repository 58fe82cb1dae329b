"""Calibration statistics, oracle side (TEST INFRASTRUCTURE ONLY).

The water-filling weight needs the per-channel key variance measured once on a
calibration sample; the rotated storage needs the eigenbasis of the
calibration key covariance, ordered by decreasing variance (yeyulingfeng.com
write-up, reverse water-filling section and the basis-choice section).

Readings: the variance is the centred population variance, accumulated in
float64 and rounded once to float32; the covariance is the centred population
covariance in float64; ``numpy.linalg.eigh`` gives the basis, columns sorted by
descending eigenvalue, eigenvalues clamped at 0.
"""
from __future__ import annotations

import numpy as np


def channel_variance(sample: np.ndarray) -> np.ndarray:
    x = np.asarray(sample, np.float64)
    mu = x.mean(axis=0)
    return ((x - mu) ** 2).mean(axis=0).astype(np.float32)


def klt_basis(sample: np.ndarray):
    """-> (U [D][D] float32, columns = eigenvectors by descending eigenvalue,
    lam [D] float32 = the variances of the rotated coordinates)."""
    x = np.asarray(sample, np.float64)
    xc = x - x.mean(axis=0)
    cov = xc.T @ xc / x.shape[0]
    lam, vec = np.linalg.eigh(cov)
    order = np.argsort(-lam, kind="stable")
    lam = np.clip(lam[order], 0.0, None)
    return vec[:, order].astype(np.float32), lam.astype(np.float32)

"""Exact-rational helpers for pinning fp32 arithmetic on tiny inputs.

fma32(a, b, c) is round-to-nearest-even of the exact a*b + c onto the float32
grid, computed with fractions -- independent of any libm or hardware fma.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def _f32(x) -> np.float32:
    return np.float32(x)


def round_f32(v: Fraction) -> np.float32:
    if v == 0:
        return np.float32(0.0)
    f = np.float32(float(v))  # within an ulp or two of the answer
    cands = {f, np.nextafter(f, np.float32(np.inf)), np.nextafter(f, np.float32(-np.inf))}
    best = None
    for c in cands:
        if not np.isfinite(c):
            continue
        d = abs(Fraction(float(c)) - v)
        if best is None or d < best[0] or (d == best[0] and (int(np.float32(c).view(np.uint32)) & 1) == 0):
            best = (d, c)
    return np.float32(best[1])


def fma32(a, b, c) -> np.float32:
    return round_f32(Fraction(float(np.float32(a))) * Fraction(float(np.float32(b))) + Fraction(float(np.float32(c))))


def mul32(a, b) -> np.float32:
    return round_f32(Fraction(float(np.float32(a))) * Fraction(float(np.float32(b))))

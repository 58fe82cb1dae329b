"""Float64 / exact-integer definitions of the method, written with numpy.

TEST INFRASTRUCTURE ONLY (see the package docstring).  These are the
real-valued definitions the fp32 contract is measured against, plus brute-force
forms used to pin the C oracle:

* ``decode_codes``     : the 4-bit codes read back from the bit planes;
* ``prefix_code`` / ``dequant``: the t-plane prefix and its mid-rise value
  (bit-plane section of the yeyulingfeng.com write-up);
* ``requant_direct``   : the t-bit mid-rise quantiser applied to x directly;
* ``scores_def``       : sum_j q_hj * k_ij in float64;
* ``contract_bound``   : the error bound the scan's fixed-point score contract
  states against ``scores_def``, and ``topk_valid``: whether a selection is
  a top-k of the definition that this bound allows;
* ``plan_bruteforce``  : exhaustive integer search of sum_j w_j 4^-t_j
  under sum_j t_j <= B (reverse water-filling section);
* ``water_level_bisect``: the smallest theta by bisection on the fp32 bit
  pattern, evaluated with fp32 arithmetic (an independent search for the same
  order statistic the C oracle takes by sorting).
"""
from __future__ import annotations

import itertools

import numpy as np


def f16_bits_to_f64(bits) -> np.ndarray:
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def decode_codes(planes: np.ndarray, n: int, channels=None) -> np.ndarray:
    """planes [D][4][nb] uint64 -> codes [D][n] (0..15), or [len(channels)][n]
    for the listed channels only."""
    if channels is not None:
        planes = planes[np.asarray(channels, np.int64)]
    D, S, nb = planes.shape
    bits = np.arange(64, dtype=np.uint64)
    codes = np.zeros((D, nb * 64), np.int64)
    for s in range(4):
        b = ((planes[:, s, :, None] >> bits[None, None, :]) & np.uint64(1)).astype(np.int64)
        codes |= b.reshape(D, nb * 64) << (3 - s)
    return codes[:, :n]


def prefix_code(codes: np.ndarray, t: int) -> np.ndarray:
    return codes >> (4 - t)


def dequant(ct, t: int, scale) -> np.ndarray:
    """(c_t - 2^(t-1) + 1/2) * 2^(4-t) * scale/8 in float64; 0 for t = 0."""
    if t == 0:
        return np.zeros(np.broadcast(ct, scale).shape)
    delta = np.asarray(scale, np.float64) / 8.0
    return (np.asarray(ct, np.float64) - 2.0 ** (t - 1) + 0.5) * 2.0 ** (4 - t) * delta


def requant_direct(x, scale, t: int) -> np.ndarray:
    """t-bit mid-rise quantiser on [-scale, scale]: cell 2^(4-t) * scale/8."""
    cell = 2.0 ** (4 - t) * (np.asarray(scale, np.float64) / 8.0)
    c = np.floor(np.asarray(x, np.float64) / cell) + 2 ** (t - 1)
    return np.clip(c, 0, 2 ** t - 1).astype(np.int64)


def pack_codes_def(keys: np.ndarray, scales_f64: np.ndarray) -> np.ndarray:
    """codes [D][n] = clip(floor(x / (scale/8)) + 8, 0, 15) for given scales
    [D][nb] (code 8 where the scale is 0)."""
    keys = np.asarray(keys, np.float64)
    n, D = keys.shape
    blk = np.arange(n) // 64
    sc = scales_f64[:, blk]  # [D][n]
    delta = sc / 8.0
    with np.errstate(divide="ignore", invalid="ignore"):
        c = np.floor(keys.T / np.where(delta > 0, delta, 1.0)) + 8
    c = np.clip(c, 0, 15)
    c = np.where(delta > 0, c, 8)
    return c.astype(np.int64)


def dequant_keys(planes, scales, n: int, depth) -> np.ndarray:
    """k_hat [D][n] in float64 for per-channel depths."""
    depth = np.asarray(depth)
    read, kr = dequant_read(planes, scales, n, depth)
    out = np.zeros((depth.shape[0], n), np.float64)
    out[read] = kr
    return out


def dequant_read(planes, scales, n: int, depth):
    """(read channels, k_hat [#read][n] float64): the prefix keys of the
    channels with depth > 0 only (what a scan reads)."""
    depth = np.asarray(depth)
    read = np.nonzero(depth)[0]
    codes = decode_codes(planes, n, read)
    sc = f16_bits_to_f64(np.asarray(scales)[read])[:, np.arange(n) // 64]
    out = np.zeros(codes.shape, np.float64)
    for r, j in enumerate(read):
        t = int(depth[j])
        out[r] = dequant(prefix_code(codes[r], t), t, sc[r])
    return read, out


def scores_def(planes, scales, n: int, depth, q_used) -> np.ndarray:
    """[G][n] float64: sum over channels of q_hj * k_hat_ij."""
    read, kr = dequant_read(planes, scales, n, depth)
    return np.asarray(q_used, np.float64)[:, read] @ kr


def contract_bound(planes, scales, n: int, depth, q_used, s_def=None) -> np.ndarray:
    """[G][n] bound on |score - s_def| that the fixed-point score contract of
    the scan states: before its final rounding a score differs from the real
    dot product by at most 15 (#read channels) 2^(E_b - 1 - sigma_h) (the
    truncated coefficients times codes of magnitude <= 15) plus
    2^-24 sum_j |q_hj k_ij| (one float32 product per coefficient); the final
    rounding to float32 adds at most 2^-24 of the magnitude.  sigma_h =
    31 - floor(log2 max_j |q_hj|) over the read channels (0 when all are 0);
    E_b = (the largest binary16 exponent field of the read channels' scales
    in block b, at least 1) - 15."""
    depth = np.asarray(depth)
    q = np.asarray(q_used, np.float64)
    read, kr = dequant_read(planes, scales, n, depth)
    if s_def is None:
        s_def = q[:, read] @ kr
    if read.size == 0:
        return np.zeros((q.shape[0], n))
    qmax = np.abs(q[:, read]).max(1)
    sigma = np.where(qmax > 0, 31 - np.floor(np.log2(np.where(qmax > 0, qmax, 1.0))), 0.0)
    ef = np.maximum(1, (np.asarray(scales)[read].astype(np.int64) >> 10) & 31).max(0)  # [nb]
    unit = np.exp2((ef - 15).astype(np.float64)[np.arange(n) // 64][None, :] - 1 - sigma[:, None])
    pre = 15 * read.size * unit + 2.0 ** -24 * (np.abs(q[:, read]) @ np.abs(kr))
    return pre + 2.0 ** -24 * (np.abs(s_def) + pre) + 2.0 ** -149


def topk_valid(s_def_row, bound_row, idx, n: int) -> bool:
    """Whether idx (k distinct tokens < n) is a valid top-k of scores known
    only to within +-bound of s_def: no token left out may be certainly above
    a token taken, i.e. min over winners of (s_def + bound) >= max over the
    others of (s_def - bound)."""
    idx = np.asarray(idx, np.int64)
    if idx.size == 0 or np.unique(idx).size != idx.size or idx.min() < 0 or idx.max() >= n:
        return False
    s = np.asarray(s_def_row[:n], np.float64)
    b = np.asarray(bound_row[:n], np.float64)
    taken = np.zeros(n, bool)
    taken[idx] = True
    if taken.all():
        return True
    return bool((s[taken] + b[taken]).min() >= (s[~taken] - b[~taken]).max())


def objective(w, t) -> float:
    """Expected squared score error up to a constant: sum_j w_j 4^-t_j."""
    w = np.asarray(w, np.float64)
    return float(np.sum(w * 4.0 ** (-np.asarray(t, np.float64))))


def plan_bruteforce(w, B: int):
    """All depth vectors in {0..4}^D with sum <= B; returns (best objective,
    list of all optimal depth vectors)."""
    w = np.asarray(w, np.float64)
    D = w.shape[0]
    cands = [t for t in itertools.product(range(5), repeat=D) if sum(t) <= B]
    vals = [objective(w, t) for t in cands]
    best = min(vals)
    return best, [t for t, v in zip(cands, vals) if v == best]


def fp32_depths(w32: np.ndarray, theta: np.float32) -> np.ndarray:
    """t_j = #{t < 4 : w_j > fl32(theta * 4^t)} in fp32 arithmetic."""
    w32 = np.asarray(w32, np.float32)
    th = np.float32(theta)
    t = np.zeros(w32.shape, np.int64)
    lvl = th
    with np.errstate(over="ignore"):
        for _ in range(4):
            t += (w32 > lvl)
            lvl = np.float32(lvl * np.float32(4.0))
    return t


def water_level_bisect(w32: np.ndarray, B: int) -> np.float32:
    """Smallest fp32 theta >= 0 with sum_j t_j(theta) <= B, searched over the
    monotone fp32 bit patterns 0 .. 0x7F800000."""
    w32 = np.asarray(w32, np.float32)
    if fp32_depths(w32, np.float32(0)).sum() <= B:
        return np.float32(0)
    lo, hi = 0, 0x7F800000
    while hi - lo > 1:
        mid = (lo + hi) // 2
        th = np.array([mid], np.uint32).view(np.float32)[0]
        if fp32_depths(w32, th).sum() <= B:
            hi = mid
        else:
            lo = mid
    return np.array([hi], np.uint32).view(np.float32)[0]


def water_level_log_bisect(w32: np.ndarray, B: int, steps: int = 30) -> float:
    """The literal form: bisection on log2(theta) over the fp32 range, keeping
    the feasible (upper) side.  Converges to within a relative 2^(-steps+~8)."""
    w32 = np.asarray(w32, np.float64)
    pos = w32[w32 > 0]
    if 4 * pos.size <= B:
        return 0.0
    lo, hi = -160.0, 130.0

    def F(lg):
        th = 2.0 ** lg
        return sum(int(np.sum(pos > th * 4.0 ** t)) for t in range(4))

    for _ in range(steps):
        mid = 0.5 * (lo + hi)
        if F(mid) <= B:
            hi = mid
        else:
            lo = mid
    return 2.0 ** hi


def topk_def(scores_row: np.ndarray, n: int, k: int) -> np.ndarray:
    """Brute force: full lexicographic sort by (-score, index)."""
    s = np.asarray(scores_row[:n], np.float64)
    s = np.where(s == 0.0, 0.0, s)
    order = np.lexsort((np.arange(n), -s))
    return order[:k].astype(np.int32)

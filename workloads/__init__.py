"""Seeded synthetic workloads for the Fathom key scan.

This module only draws random inputs -- keys, queries, calibration samples,
mixing matrices -- and names the workload shapes.  It holds none of the
method's arithmetic, so that the HIP library's tests and the CPU oracle can
both be fed from it.

Every stream is numpy PCG64 seeded with SeedSequence([20260915, layer,
kv_head, stream]), streams 0 = channel scales, 1 = keys, 2 = queries,
3 = planted positions, 4 = calibration sample, 5 = mixing matrix,
6 = values (for attention-output error measurements).  Large key
tensors (131k and 1M tokens x 288 pairs) are drawn on the GPU with torch's
Philox generator seeded from the same SeedSequence; small ones on the host.

Workloads stand in for the pages' Qwen3-8B-shaped decode step (36 layers x 8
KV heads, D = 128, G = 4 query heads per KV head); the pages measured real
model keys up to 128k and synthetic KV above that.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

BASE_SEED = 20260915
S_SCALES, S_KEYS, S_QUERIES, S_PLANTED, S_CALIB, S_MIX, S_VALUES = range(7)
CALIB_KEYS = 8192


@dataclass(frozen=True)
class Workload:
    name: str
    layers: int
    kv_heads: int
    n: int
    G: int = 4
    D: int = 128
    budget: int = 48
    k: int = 512
    key_dtype: str = "bf16"      # "f32" | "bf16"
    sigma_log: float = 0.3       # channel scale s_j = exp(sigma_log * z)
    outliers: int = 0            # channels multiplied by 8 (tiny workload)
    planted: int = 0             # planted keys per head (tiny workload)
    heavy_q: int = 8             # per-head channels with largest |q| scaled x5
    mixed: bool = False          # keys mixed by a random orthogonal matrix
    rotated: bool = False        # index stored in the calibration KLT basis
    host_resident: bool = False  # index in mapped pinned host memory
    sweep: tuple = field(default=())

    @property
    def P(self) -> int:
        return self.layers * self.kv_heads

    @property
    def nb(self) -> int:
        return (self.n + 63) // 64

    def pair(self, p: int):
        return divmod(p, self.kv_heads)


WORKLOADS = {
    # 1 layer, 1 KV head, n=4096, fp32 keys with 4 outlier channels (x8) and
    # 16 keys per head planted at 3x that head's query; B=48, k=64.
    "tiny": Workload("tiny", 1, 1, 4096, k=64, key_dtype="f32", sigma_log=0.5,
                     outliers=4, planted=16, heavy_q=0),
    # one Qwen3-8B-shaped layer at 32k: flat (QK-norm-like) channel scales,
    # queries with 8 heavy channels per head.
    "qwen32k": Workload("qwen32k", 1, 8, 32768),
    # all 36 x 8 pairs at 131k, plus the budget sweep and the 136-bit baseline.
    "sweep131k": Workload("sweep131k", 36, 8, 131072, sweep=(32, 48, 68, 92, 136)),
    # one decode step at 1M tokens over 288 pairs, Llama-like wide channel
    # scales (no QK-norm).
    "long1m": Workload("long1m", 36, 8, 1 << 20, sigma_log=1.0),
    # the same step with the index in pinned host memory, keys mixed by a
    # random orthogonal matrix and stored in the calibration KLT basis.
    "host1m_klt": Workload("host1m_klt", 36, 8, 1 << 20, sigma_log=1.0, mixed=True,
                           rotated=True, host_resident=True),
}


def rng(layer: int, kv: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([BASE_SEED, layer, kv, stream])))


def torch_seed(layer: int, kv: int, stream: int) -> int:
    st = np.random.SeedSequence([BASE_SEED, layer, kv, stream]).generate_state(2, np.uint32)
    return int(st[0]) | (int(st[1] & 0x7FFFFFFF) << 32)


def to_bf16_exact(x: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bfloat16 (ties to even); returned as the
    float32 values that bfloat16 represents exactly."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (r.astype(np.uint32) << 16).view(np.float32)


def bf16_bits(x_exact: np.ndarray) -> np.ndarray:
    """float32 values that are exact bf16 -> their uint16 bit patterns."""
    return (np.ascontiguousarray(x_exact, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def channel_scales(w: Workload, p: int) -> np.ndarray:
    layer, kv = w.pair(p)
    g = rng(layer, kv, S_SCALES)
    s = np.exp(w.sigma_log * g.standard_normal(w.D))
    if w.outliers:
        s[g.choice(w.D, w.outliers, replace=False)] *= 8.0
    return s.astype(np.float32)


def mixing(w: Workload, p: int) -> np.ndarray | None:
    """Random orthogonal D x D matrix (QR of a Gaussian, signs fixed)."""
    if not w.mixed:
        return None
    layer, kv = w.pair(p)
    a = rng(layer, kv, S_MIX).standard_normal((w.D, w.D))
    qm, r = np.linalg.qr(a)
    return (qm * np.sign(np.diag(r))).astype(np.float32)


def _raw_keys(w: Workload, p: int, n: int, stream: int) -> np.ndarray:
    layer, kv = w.pair(p)
    s = channel_scales(w, p)
    z = rng(layer, kv, stream).standard_normal((n, w.D), dtype=np.float32)
    x = z * s[None, :]
    m = mixing(w, p)
    if m is not None:
        x = x @ m.T
    return x.astype(np.float32)


def queries(w: Workload, p: int) -> np.ndarray:
    layer, kv = w.pair(p)
    q = rng(layer, kv, S_QUERIES).standard_normal((w.G, w.D)).astype(np.float32)
    if w.heavy_q:
        for h in range(w.G):
            top = np.argsort(-np.abs(q[h]), kind="stable")[: w.heavy_q]
            q[h, top] *= 5.0
    return q


def keys_host(w: Workload, p: int, n: int | None = None) -> np.ndarray:
    """Keys of one pair on the host, [n][D] float32 (bf16-exact for bf16
    workloads), planted keys included."""
    n = w.n if n is None else n
    x = _raw_keys(w, p, n, S_KEYS)
    if w.planted:
        layer, kv = w.pair(p)
        q = queries(w, p)
        pos = rng(layer, kv, S_PLANTED).choice(n, w.G * w.planted, replace=False)
        for h in range(w.G):
            x[pos[h * w.planted:(h + 1) * w.planted]] = 3.0 * q[h]
    if w.key_dtype == "bf16":
        x = to_bf16_exact(x)
    return x


def planted_positions(w: Workload, p: int, n: int | None = None) -> np.ndarray:
    n = w.n if n is None else n
    layer, kv = w.pair(p)
    return rng(layer, kv, S_PLANTED).choice(n, w.G * w.planted, replace=False).reshape(w.G, w.planted)


def values_host(w: Workload, p: int, n: int | None = None) -> np.ndarray:
    """Values of one pair, [n][D] float32 N(0, 1) (bf16-exact for bf16
    workloads): only used to measure attention-output error."""
    n = w.n if n is None else n
    layer, kv = w.pair(p)
    v = rng(layer, kv, S_VALUES).standard_normal((n, w.D), dtype=np.float32)
    return to_bf16_exact(v) if w.key_dtype == "bf16" else v


def calibration_sample(w: Workload, p: int) -> np.ndarray:
    """A separate 8192-key sample of the same distribution (nothing planted)."""
    x = _raw_keys(w, p, CALIB_KEYS, S_CALIB)
    if w.key_dtype == "bf16":
        x = to_bf16_exact(x)
    return x


def keys_device(w: Workload, pairs, device="cuda", n: int | None = None):
    """Keys of several pairs drawn on the GPU: torch tensor [len(pairs)][n][D]
    (bfloat16 or float32).  Philox streams seeded per pair."""
    import torch

    n = w.n if n is None else n
    dt = torch.bfloat16 if w.key_dtype == "bf16" else torch.float32
    out = torch.empty((len(pairs), n, w.D), dtype=dt, device=device)
    gen = torch.Generator(device=device)
    for i, p in enumerate(pairs):
        layer, kv = w.pair(p)
        gen.manual_seed(torch_seed(layer, kv, S_KEYS))
        s = torch.from_numpy(channel_scales(w, p)).to(device)
        z = torch.randn((n, w.D), generator=gen, device=device, dtype=torch.float32)
        z.mul_(s)
        m = mixing(w, p)
        if m is not None:
            z = z @ torch.from_numpy(m).to(device).T.contiguous()
        out[i].copy_(z)
        del z
    return out

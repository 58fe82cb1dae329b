"""Fathom CPU oracle -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library
(``sparse_attention_key_amd``) never imports it, and it imports nothing from
the product.  It holds two independent descriptions of the method:

* ``fathom_oracle.c`` (loaded through ctypes): the plain procedure -- pack,
  plan, the fixed-point score contract (exact integer sums per block, one
  final rounding), top-k, union -- one (layer, KV head) pair per call;
* ``ref64`` (numpy, float64): the real-valued definitions used for the
  tolerance checks (dequantised prefix keys and the exact score sum).

Source of the method: the yeyulingfeng.com write-up of "Fathom: Per-Query Read
Depth for Sparse Decoding over Offloaded KV Caches" (arXiv 2609.17652),
sections on bit planes (method one) and reverse water-filling (method two),
and the bit-plane figure on the paotong.dev page.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fathom_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liborc.so")

PLAN_WATERFILL = 0
PLAN_TOPR = 1
PLAN_UNIFORM = 2


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (no fp contraction: every fma is explicit)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
             "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i64, i32 = ctypes.c_int64, ctypes.c_int
        L.orc_f32_to_f16.argtypes = [ctypes.c_float]
        L.orc_f32_to_f16.restype = ctypes.c_uint16
        L.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_f16_to_f32.restype = ctypes.c_float
        L.orc_code.argtypes = [ctypes.c_float, ctypes.c_uint16]
        L.orc_code.restype = i32
        L.orc_pack.argtypes = [P, i64, i32, P, P, P]
        L.orc_pack.restype = None
        L.orc_prefix_code.argtypes = [P, i64, i32, i64, i32]
        L.orc_prefix_code.restype = i32
        L.orc_dequant.argtypes = [i32, i32, ctypes.c_uint16]
        L.orc_dequant.restype = ctypes.c_float
        L.orc_query_used.argtypes = [P, P, i32, i32, P]
        L.orc_query_used.restype = None
        L.orc_importance.argtypes = [P, P, i32, i32, P]
        L.orc_importance.restype = None
        L.orc_depth_at.argtypes = [ctypes.c_float, ctypes.c_float]
        L.orc_depth_at.restype = i32
        L.orc_water_level.argtypes = [P, i32, i32]
        L.orc_water_level.restype = ctypes.c_float
        L.orc_plan.argtypes = [P, P, P, i32, i32, i32, i32, P, P]
        L.orc_plan.restype = ctypes.c_float
        L.orc_scores.argtypes = [P, P, i64, i32, P, P, i32, P]
        L.orc_scores.restype = None
        L.orc_scores_f64.argtypes = [P, P, i64, i32, P, P, i32, P]
        L.orc_scores_f64.restype = None
        L.orc_topk.argtypes = [P, i64, i32, P, P]
        L.orc_topk.restype = None
        L.orc_union.argtypes = [P, i32, i32, P]
        L.orc_union.restype = i32
        L.orc_step.argtypes = [P, P, i64, i32, P, P, P, i32, i32, i32, i32, P, P, P, P, P]
        L.orc_step.restype = i32
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dt):
    return None if a is None else np.ascontiguousarray(a, dtype=dt)


# ---------------------------------------------------------------- one pair

def f32_to_f16_bits(x: float) -> int:
    return int(lib().orc_f32_to_f16(float(x)))


def f16_bits_to_f32(h: int) -> float:
    return float(lib().orc_f16_to_f32(int(h)))


def code(x: float, scale_bits: int) -> int:
    return int(lib().orc_code(float(x), int(scale_bits)))


def dequant(ct: int, t: int, scale_bits: int) -> float:
    return float(lib().orc_dequant(int(ct), int(t), int(scale_bits)))


def pack(keys: np.ndarray, rot: np.ndarray | None = None):
    """keys [n][D] (float32; bf16 inputs are widened exactly first) ->
    (planes [D][4][nb] uint64, scales [D][nb] uint16 fp16 bits)."""
    keys = _c(keys, np.float32)
    rot = _c(rot, np.float32)
    n, D = keys.shape
    nb = (n + 63) // 64
    planes = np.zeros((D, 4, nb), np.uint64)
    scales = np.zeros((D, nb), np.uint16)
    lib().orc_pack(_p(keys), n, D, _p(rot), _p(planes), _p(scales))
    return planes, scales


def query_used(q, rot=None):
    q = _c(q, np.float32)
    G, D = q.shape
    out = np.zeros((G, D), np.float32)
    lib().orc_query_used(_p(q), _p(_c(rot, np.float32)), G, D, _p(out))
    return out


def importance(q_used, sigma2):
    q_used = _c(q_used, np.float32)
    G, D = q_used.shape
    w = np.zeros(D, np.float32)
    lib().orc_importance(_p(q_used), _p(_c(sigma2, np.float32)), G, D, _p(w))
    return w


def water_level(w, B: int) -> float:
    w = _c(w, np.float32)
    return float(lib().orc_water_level(_p(w), w.shape[0], int(B)))


def depth_at(w: float, theta: float) -> int:
    return int(lib().orc_depth_at(float(w), float(theta)))


def plan(q, sigma2, budget: int, mode: int = PLAN_WATERFILL, rot=None):
    """-> (depth [D] uint8, theta float, q_used [G][D] float32)."""
    q = _c(q, np.float32)
    G, D = q.shape
    depth = np.zeros(D, np.uint8)
    q_used = np.zeros((G, D), np.float32)
    theta = lib().orc_plan(_p(q), _p(_c(sigma2, np.float32)), _p(_c(rot, np.float32)),
                           G, D, int(budget), int(mode), _p(depth), _p(q_used))
    return depth, float(theta), q_used


def scores(planes, scales, n: int, depth, q_used):
    """Scores under the fixed-point contract (exact integer sum per block,
    one final rounding to float32); tokens >= n are -inf."""
    planes = _c(planes, np.uint64)
    scales = _c(scales, np.uint16)
    depth = _c(depth, np.uint8)
    q_used = _c(q_used, np.float32)
    G, D = q_used.shape
    nb = (n + 63) // 64
    out = np.zeros((G, nb * 64), np.float32)
    lib().orc_scores(_p(planes), _p(scales), n, D, _p(depth), _p(q_used), G, _p(out))
    return out


def scores_f64(planes, scales, n: int, depth, q_used):
    planes = _c(planes, np.uint64)
    scales = _c(scales, np.uint16)
    depth = _c(depth, np.uint8)
    q_used = _c(q_used, np.float32)
    G, D = q_used.shape
    out = np.zeros((G, n), np.float64)
    lib().orc_scores_f64(_p(planes), _p(scales), n, D, _p(depth), _p(q_used), G, _p(out))
    return out


def topk(scores_row, n: int, k: int):
    """Top-k of one head -> (idx [k] int32, val [k] float32)."""
    s = _c(scores_row, np.float32)
    idx = np.zeros(k, np.int32)
    val = np.zeros(k, np.float32)
    lib().orc_topk(_p(s), n, int(k), _p(idx), _p(val))
    return idx, val


def union(idx_gk):
    idx = _c(idx_gk, np.int32)
    G, k = idx.shape
    out = np.zeros(G * k, np.int32)
    ln = lib().orc_union(_p(idx), G, k, _p(out))
    return out, int(ln)


def step(planes, scales, n, q, sigma2, budget, k, mode=PLAN_WATERFILL, rot=None):
    """plan + scores + per-head top-k + union for one pair."""
    planes = _c(planes, np.uint64)
    scales = _c(scales, np.uint16)
    q = _c(q, np.float32)
    G, D = q.shape
    nb = (n + 63) // 64
    depth = np.zeros(D, np.uint8)
    q_used = np.zeros((G, D), np.float32)
    scores = np.zeros((G, nb * 64), np.float32)
    tk = np.zeros((G, k), np.int32)
    un = np.zeros(G * k, np.int32)
    ln = lib().orc_step(_p(planes), _p(scales), n, D, _p(q), _p(_c(sigma2, np.float32)),
                        _p(_c(rot, np.float32)), G, int(budget), int(mode), int(k),
                        _p(depth), _p(q_used), _p(scores), _p(tk), _p(un))
    return dict(depth=depth, q_used=q_used, scores=scores, topk=tk, union=un, union_len=int(ln))


def gather_rows(table: np.ndarray, union_idx: np.ndarray, union_len: np.ndarray, out: np.ndarray):
    """Winner-row fetch by definition: out[p][r] = table[p][union_idx[p][r]]
    for r < union_len[p] and valid indices (table [P][rows][...] or a shared
    [rows][...] table); other rows of `out` are left as they are."""
    out = out.copy()
    for p in range(union_idx.shape[0]):
        t = table if table.ndim == out.ndim - 1 else table[p]
        for r in range(int(union_len[p])):
            i = int(union_idx[p, r])
            if 0 <= i < t.shape[0]:
                out[p, r] = t[i]
    return out


from . import ref64  # noqa: E402,F401  (float64 definitions)
from . import calib  # noqa: E402,F401  (calibration statistics)

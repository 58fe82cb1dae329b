"""Shared helpers for the GPU parity tests (host <-> device plumbing only)."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


def u64(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint64)


def u16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def bf16_dev(x_exact: np.ndarray) -> torch.Tensor:
    """float32 array holding bf16-exact values -> bfloat16 device tensor."""
    return torch.from_numpy(np.ascontiguousarray(x_exact, np.float32)).to(torch.bfloat16).cuda()


def score_tol(ref64: np.ndarray, q_used: np.ndarray, scales_bits: np.ndarray) -> np.ndarray:
    """|s - s_def| bound: 1e-5 relative + 1e-6 * ||q_h||_1 * max scale."""
    smax = float(np.asarray(scales_bits, np.uint16).view(np.float16).astype(np.float64).max())
    return 1e-5 * np.abs(ref64) + 1e-6 * np.abs(q_used.astype(np.float64)).sum(-1, keepdims=True) * smax


def assert_selection_valid(orc, planes, scales, n, depth, q_used, idx):
    """The GPU's per-head selections idx [G][k] are a valid top-k of the plain
    float64 score definition (query times prefix-dequantised keys) within
    the error bound the fixed-point score contract states (oracle.ref64)."""
    s_def = orc.ref64.scores_def(planes, scales, n, depth, q_used)
    bnd = orc.ref64.contract_bound(planes, scales, n, depth, q_used, s_def=s_def)
    for h in range(idx.shape[0]):
        assert orc.ref64.topk_valid(s_def[h], bnd[h], idx[h], n), f"head {h}: not a top-k of the definition"

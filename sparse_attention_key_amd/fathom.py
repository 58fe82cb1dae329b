"""Python binding of libfathom.so (the gfx950 HIP library, C ABI in
include/fathom.h).

Argument marshalling only: torch supplies device memory and the current HIP
stream; every step of the path runs in the library's kernels.  There is no
fallback: if the library is not built this module raises on first use.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfathom.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "fathom.h")

OK = 0
ERR_ARG, ERR_SHAPE, ERR_ALIGN, ERR_WORKSPACE, ERR_UNSUPPORTED, ERR_HIP = -1, -2, -3, -4, -5, -6
DTYPE_F32, DTYPE_BF16 = 0, 1
PLAN_WATERFILL, PLAN_TOPR, PLAN_UNIFORM = 0, 1, 2
MAX_K = 4096


class FathomError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libfathom.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise FathomError("load", ERR_HIP,
                              f"{LIB_PATH} is missing; build it with python -m sparse_attention_key_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.fathom_abi_version.argtypes, L.fathom_abi_version.restype = [], ctypes.c_int
        L.fathom_strerror.argtypes, L.fathom_strerror.restype = [ctypes.c_int], ctypes.c_char_p
        L.fathom_pack.argtypes = [P, i32, i32, i64, i32, P, P, P, P]
        L.fathom_pack_range.argtypes = [P, i32, i32, i64, i64, i32, P, P, P, i64, P]
        L.fathom_plan.argtypes = [P, P, P, i32, i32, i32, i32, i32, P, P, P, P, P, P]
        L.fathom_scan.argtypes = [P, P, i32, i32, i64, i64, P, P, P, P, i32, P, P]
        L.fathom_topk_workspace_bytes.argtypes = [i32, i32, i64, i32]
        L.fathom_topk_workspace_bytes.restype = sz
        L.fathom_topk.argtypes = [P, i32, i32, i64, i32, P, P, P, P, P, sz, P]
        L.fathom_scan_topk_workspace_bytes.argtypes = [i32, i32, i64, i32]
        L.fathom_scan_topk_workspace_bytes.restype = sz
        L.fathom_scan_topk.argtypes = [P, P, i32, i32, i64, i64, P, P, P, P, i32, i32, P, P, P, P, P, sz, P]
        L.fathom_scan_topk_stage.argtypes = [i32] + L.fathom_scan_topk.argtypes
        L.fathom_scan_topk_noalloc.argtypes = L.fathom_scan_topk.argtypes[:16] + [P]
        L.fathom_read_probe.argtypes = [P, sz, P, P]
        L.fathom_gather_rows.argtypes = [P, i64, i64, i64, i32, P, P, i32, P, P]
        L.fathom_gather_rows.restype = ctypes.c_int
        L.fathom_calib_workspace_bytes.argtypes = [i32, i64, i32]
        L.fathom_calib_workspace_bytes.restype = sz
        L.fathom_calib_covariance.argtypes = [P, i32, i32, i64, i32, P, P, P, sz, P]
        L.fathom_calib_covariance.restype = ctypes.c_int
        L.fathom_calib_basis.argtypes = [P, i32, i32, P, P, P]
        L.fathom_calib_basis.restype = ctypes.c_int
        L.fathom_read_probe.restype = ctypes.c_int
        for f in (L.fathom_pack, L.fathom_pack_range, L.fathom_plan, L.fathom_scan, L.fathom_topk,
                  L.fathom_scan_topk, L.fathom_scan_topk_stage, L.fathom_scan_topk_noalloc):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


def declared_symbols() -> list[str]:
    """Names of the entry points declared in include/fathom.h."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(fathom_\w+)\s*\(", text, re.M)))


def _check(fn: str, rc: int):
    if rc != OK:
        raise FathomError(fn, rc, lib().fathom_strerror(rc).decode())


def _ptr(t):
    """Device address of a dense device tensor, or a raw address given as an
    int (e.g. a mapped pinned host buffer).  Strided or host tensors are
    refused: the library reads every array as dense row-major memory."""
    if t is None:
        return None
    if isinstance(t, int):
        return ctypes.c_void_p(t)
    if not t.is_cuda:
        raise ValueError("fathom: tensor arguments must live in device memory")
    if not t.is_contiguous():
        raise ValueError(f"fathom: tensor of shape {tuple(t.shape)} is not contiguous; "
                         "the entry points read dense row-major arrays")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def nblocks(n: int) -> int:
    return (n + 63) // 64


def _nb_cap(planes, nb_cap):
    """Blocks per index row: given, else the last dimension of a [P][D][4][L]
    planes tensor, else 0 (a dense index)."""
    if nb_cap is not None:
        return int(nb_cap)
    if isinstance(planes, torch.Tensor) and planes.dim() == 4:
        return int(planes.shape[-1])
    return 0


# ------------------------------------------------------------------- pack

def pack_into(keys, planes, scales, rot=None, stream=None):
    """keys [P][n][D] float32|bfloat16 -> planes [P][D][4][nb] (int64 storage
    of uint64 words), scales [P][D][nb] (int16 storage of fp16 bits)."""
    P, n, D = keys.shape
    dt = {torch.float32: DTYPE_F32, torch.bfloat16: DTYPE_BF16}[keys.dtype]
    _check("fathom_pack", lib().fathom_pack(_ptr(keys), dt, P, n, D, _ptr(rot), _ptr(planes),
                                            _ptr(scales), _stream(stream)))


def pack_range(keys, tok0: int, planes, scales, rot=None, stream=None):
    """Pack keys [P][m][D] as tokens tok0 .. tok0+m-1 (tok0 a multiple of 64)
    into an index planes [P][D][4][nb_cap], scales [P][D][nb_cap]; other
    blocks are left as they are (appends repack the tail block)."""
    P, m, D = keys.shape
    dt = {torch.float32: DTYPE_F32, torch.bfloat16: DTYPE_BF16}[keys.dtype]
    _check("fathom_pack_range", lib().fathom_pack_range(
        _ptr(keys), dt, P, int(tok0), m, D, _ptr(rot), _ptr(planes), _ptr(scales),
        int(planes.shape[-1]), _stream(stream)))


def pack(keys, rot=None, stream=None):
    P, n, D = keys.shape
    nb = nblocks(n)
    planes = torch.empty((P, D, 4, nb), dtype=torch.int64, device=keys.device)
    scales = torch.empty((P, D, nb), dtype=torch.int16, device=keys.device)
    pack_into(keys, planes, scales, rot, stream)
    return planes, scales


# ------------------------------------------------------------------- plan

class Plan:
    """Device buffers of a read plan for P pairs."""

    def __init__(self, P: int, G: int, D: int, device="cuda"):
        self.P, self.G, self.D = P, G, D
        self.depth = torch.empty((P, D), dtype=torch.uint8, device=device)
        self.active = torch.empty((P, D), dtype=torch.int16, device=device)
        self.n_active = torch.empty((P,), dtype=torch.int32, device=device)
        self.theta = torch.empty((P,), dtype=torch.float32, device=device)
        self.q_used = torch.empty((P, G, D), dtype=torch.float32, device=device)


def plan_into(plan: Plan, q, sigma2, budget: int, mode: int = PLAN_WATERFILL, rot=None, stream=None):
    P, G, D = q.shape
    _check("fathom_plan", lib().fathom_plan(
        _ptr(q), _ptr(sigma2), _ptr(rot), P, G, D, int(budget), int(mode), _ptr(plan.depth),
        _ptr(plan.active), _ptr(plan.n_active), _ptr(plan.theta), _ptr(plan.q_used), _stream(stream)))
    return plan


def plan(q, sigma2, budget: int, mode: int = PLAN_WATERFILL, rot=None, stream=None) -> Plan:
    P, G, D = q.shape
    return plan_into(Plan(P, G, D, q.device), q, sigma2, budget, mode, rot, stream)


# ------------------------------------------------------------------- scan

def scan_into(planes, scales, n: int, pl: Plan, scores, stream=None, nb_cap=None):
    P, D = pl.P, pl.D
    _check("fathom_scan", lib().fathom_scan(
        _ptr(planes), _ptr(scales), P, D, int(n), _nb_cap(planes, nb_cap), _ptr(pl.depth),
        _ptr(pl.active), _ptr(pl.n_active), _ptr(pl.q_used), pl.G, _ptr(scores), _stream(stream)))


def scan(planes, scales, n: int, pl: Plan, stream=None, nb_cap=None):
    scores = torch.empty((pl.P, pl.G, nblocks(n) * 64), dtype=torch.float32, device=pl.q_used.device)
    scan_into(planes, scales, n, pl, scores, stream, nb_cap)
    return scores


# ------------------------------------------------------------------ top-k

def topk_workspace_bytes(P: int, G: int, n: int, k: int) -> int:
    return int(lib().fathom_topk_workspace_bytes(P, G, int(n), int(k)))


def scan_topk_workspace_bytes(P: int, G: int, n: int, k: int) -> int:
    return int(lib().fathom_scan_topk_workspace_bytes(P, G, int(n), int(k)))


class TopkOut:
    def __init__(self, P: int, G: int, n: int, k: int, device="cuda", with_values=True,
                 fused: bool = False, workspace: bool = True):
        self.P, self.G, self.n, self.k = P, G, n, k
        self.idx = torch.empty((P, G, k), dtype=torch.int32, device=device)
        self.val = torch.empty((P, G, k), dtype=torch.float32, device=device) if with_values else None
        self.union = torch.empty((P, G * k), dtype=torch.int32, device=device)
        self.union_len = torch.empty((P,), dtype=torch.int32, device=device)
        self.ws = None  # workspace=False: outputs only (for scan_topk_noalloc_into)
        if workspace:
            ws_fn = scan_topk_workspace_bytes if fused else topk_workspace_bytes
            nbytes = max(ws_fn(P, G, n, k), 16)
            self.ws = torch.empty((nbytes + 15) // 16 * 16, dtype=torch.uint8, device=device)


def topk_into(scores, n: int, out: TopkOut, stream=None):
    P, G, _ = scores.shape
    _check("fathom_topk", lib().fathom_topk(
        _ptr(scores), P, G, int(n), out.k, _ptr(out.idx), _ptr(out.val), _ptr(out.union),
        _ptr(out.union_len), _ptr(out.ws), out.ws.numel(), _stream(stream)))
    return out


def topk(scores, n: int, k: int, stream=None) -> TopkOut:
    P, G, _ = scores.shape
    return topk_into(scores, n, TopkOut(P, G, n, k, scores.device), stream)


# ------------------------------------------------------- fused scan + top-k

def scan_topk_into(planes, scales, n: int, pl: Plan, out: TopkOut, stream=None, nb_cap=None):
    """Scores, top-k and union of every pair without materialising scores;
    `out` must be a TopkOut(..., fused=True)."""
    _check("fathom_scan_topk", lib().fathom_scan_topk(
        _ptr(planes), _ptr(scales), pl.P, pl.D, int(n), _nb_cap(planes, nb_cap), _ptr(pl.depth),
        _ptr(pl.active),
        _ptr(pl.n_active), _ptr(pl.q_used), pl.G, out.k, _ptr(out.idx), _ptr(out.val), _ptr(out.union),
        _ptr(out.union_len), _ptr(out.ws), out.ws.numel(), _stream(stream)))
    return out


def scan_topk(planes, scales, n: int, pl: Plan, k: int, stream=None, nb_cap=None) -> TopkOut:
    out = TopkOut(pl.P, pl.G, n, k, pl.q_used.device, fused=True)
    return scan_topk_into(planes, scales, n, pl, out, stream, nb_cap)


def scan_topk_noalloc_into(planes, scales, n: int, pl: Plan, out: TopkOut, stream=None, nb_cap=None):
    """scan_topk_into with the library's fixed per-GPU scratch as workspace
    (no device allocation; out.ws is not used, so `out` may be a
    TopkOut(..., workspace=False)).  Calls that overlap on one GPU race."""
    _check("fathom_scan_topk_noalloc", lib().fathom_scan_topk_noalloc(
        _ptr(planes), _ptr(scales), pl.P, pl.D, int(n), _nb_cap(planes, nb_cap), _ptr(pl.depth),
        _ptr(pl.active), _ptr(pl.n_active), _ptr(pl.q_used), pl.G, out.k, _ptr(out.idx), _ptr(out.val),
        _ptr(out.union), _ptr(out.union_len), _stream(stream)))
    return out


def scan_topk_stage(stage: int, planes, scales, n: int, pl: Plan, out: TopkOut, stream=None,
                    nb_cap=None):
    """One stage (1 threshold, 2 filtered scan, 3 select + union) of scan_topk_into."""
    _check("fathom_scan_topk_stage", lib().fathom_scan_topk_stage(
        int(stage), _ptr(planes), _ptr(scales), pl.P, pl.D, int(n), _nb_cap(planes, nb_cap),
        _ptr(pl.depth), _ptr(pl.active),
        _ptr(pl.n_active), _ptr(pl.q_used), pl.G, out.k, _ptr(out.idx), _ptr(out.val), _ptr(out.union),
        _ptr(out.union_len), _ptr(out.ws), out.ws.numel(), _stream(stream)))
    return out


def read_probe(src, nbytes: int, sink, stream=None):
    """Stream nbytes of src once (bandwidth probe; see fathom_read_probe)."""
    _check("fathom_read_probe", lib().fathom_read_probe(_ptr(src), int(nbytes), _ptr(sink), _stream(stream)))


def gather_rows(table, table_rows: int, row_bytes: int, pair_stride_rows: int, union, union_len, out,
                stream=None):
    """Fetch the union rows of every pair from a row table (device memory or
    mapped host memory given as an int address) into out [P][cap][row_bytes]."""
    P, cap = union.shape
    _check("fathom_gather_rows", lib().fathom_gather_rows(
        _ptr(table), int(table_rows), int(row_bytes), int(pair_stride_rows), P, _ptr(union),
        _ptr(union_len), cap, _ptr(out), _stream(stream)))
    return out


# ------------------------------------------------------------ calibration

def calib_workspace_bytes(P: int, m: int, D: int) -> int:
    return int(lib().fathom_calib_workspace_bytes(P, int(m), D))


def calib_covariance(keys, with_cov: bool = True, stream=None):
    """keys [P][m][D] float32|bfloat16 (calibration or prefill keys) ->
    (cov [P][D][D] float64 centred population covariance or None,
     var [P][D] float32 channel variances)."""
    P, m, D = keys.shape
    dt = {torch.float32: DTYPE_F32, torch.bfloat16: DTYPE_BF16}[keys.dtype]
    cov = torch.empty((P, D, D), dtype=torch.float64, device=keys.device) if with_cov else None
    var = torch.empty((P, D), dtype=torch.float32, device=keys.device)
    nbytes = calib_workspace_bytes(P, m, D)
    ws = torch.empty((nbytes + 15) // 16 * 16, dtype=torch.uint8, device=keys.device)
    _check("fathom_calib_covariance", lib().fathom_calib_covariance(
        _ptr(keys), dt, P, int(m), D, _ptr(cov), _ptr(var), _ptr(ws), ws.numel(), _stream(stream)))
    return cov, var


def calib_basis(cov, stream=None):
    """cov [P][D][D] float64 -> (U [P][D][D] float32, columns the eigenvectors
    by descending eigenvalue, lam [P][D] float32 eigenvalues clamped at 0)."""
    P, D, _ = cov.shape
    U = torch.empty((P, D, D), dtype=torch.float32, device=cov.device)
    lam = torch.empty((P, D), dtype=torch.float32, device=cov.device)
    _check("fathom_calib_basis", lib().fathom_calib_basis(_ptr(cov), P, D, _ptr(U), _ptr(lam),
                                                          _stream(stream)))
    return U, lam

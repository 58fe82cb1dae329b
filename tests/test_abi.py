"""The C-ABI library loads without a GPU, exports every declared entry point,
and rejects bad arguments on the host before touching HIP."""
import ctypes

import pytest

from sparse_attention_key_amd import fathom as F


@pytest.fixture(scope="module")
def L():
    return F.lib()


def test_exports_every_declared_symbol(L):
    names = F.declared_symbols()
    assert {"fathom_pack", "fathom_plan", "fathom_scan", "fathom_topk"} <= set(names)
    for name in names:
        assert hasattr(L, name), name


def test_version_and_strerror(L):
    assert L.fathom_abi_version() == 2
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert L.fathom_strerror(code)
    assert L.fathom_strerror(-99) == b"unknown status"


A = ctypes.c_void_p(16 * 4096)      # aligned dummy (never dereferenced)
MIS = ctypes.c_void_p(16 * 4096 + 4)  # misaligned dummy


def test_pack_validation(L):
    assert L.fathom_pack(None, 0, 1, 64, 128, None, A, A, None) == F.ERR_ARG
    assert L.fathom_pack(A, 7, 1, 64, 128, None, A, A, None) == F.ERR_ARG
    assert L.fathom_pack(A, 0, 0, 64, 128, None, A, A, None) == F.ERR_SHAPE
    assert L.fathom_pack(A, 0, 1, 0, 128, None, A, A, None) == F.ERR_SHAPE
    assert L.fathom_pack(A, 0, 1, 64, 129, None, A, A, None) == F.ERR_SHAPE
    assert L.fathom_pack(A, 0, 1, 1 << 31, 128, None, A, A, None) == F.ERR_SHAPE
    assert L.fathom_pack(A, 0, 65536, 64, 128, None, A, A, None) == F.ERR_SHAPE
    assert L.fathom_pack(MIS, 0, 1, 64, 128, None, A, A, None) == F.ERR_ALIGN
    assert L.fathom_pack(A, 1, 1, 64, 128, MIS, A, A, None) == F.ERR_ALIGN


def test_plan_validation(L):
    args = lambda **kw: [kw.get("q", A), A, kw.get("rot", None), kw.get("P", 1), kw.get("G", 4),
                         kw.get("D", 128), kw.get("B", 48), kw.get("mode", 0), A, A, A, A, A, None]
    assert L.fathom_plan(*args(q=None)) == F.ERR_ARG
    assert L.fathom_plan(*args(G=9)) == F.ERR_SHAPE
    assert L.fathom_plan(*args(G=0)) == F.ERR_SHAPE
    assert L.fathom_plan(*args(D=0)) == F.ERR_SHAPE
    assert L.fathom_plan(*args(B=-1)) == F.ERR_ARG
    assert L.fathom_plan(*args(B=513)) == F.ERR_ARG
    assert L.fathom_plan(*args(B=129, mode=1)) == F.ERR_ARG
    assert L.fathom_plan(*args(B=5, mode=2)) == F.ERR_ARG
    assert L.fathom_plan(*args(mode=3)) == F.ERR_ARG
    assert L.fathom_plan(*args(q=MIS)) == F.ERR_ALIGN
    assert L.fathom_plan(*args(rot=MIS)) == F.ERR_ALIGN


def test_scan_validation(L):
    # planes, scales, P, D, n, nb_cap, depth, active, n_active, q_used, G, scores, stream
    base = [A, A, 1, 128, 4096, 0, A, A, A, A, 4, A, None]

    def with_(i, v):
        b = list(base)
        b[i] = v
        return b
    assert L.fathom_scan(*with_(11, None)) == F.ERR_ARG
    assert L.fathom_scan(*with_(10, 9)) == F.ERR_SHAPE
    assert L.fathom_scan(*with_(4, 0)) == F.ERR_SHAPE
    assert L.fathom_scan(*with_(2, 65536)) == F.ERR_SHAPE
    assert L.fathom_scan(*with_(5, 63)) == F.ERR_SHAPE       # 4096 tokens need 64 blocks per row
    assert L.fathom_scan(*with_(5, -1)) == F.ERR_SHAPE
    assert L.fathom_scan(*with_(5, 1 << 26)) == F.ERR_SHAPE
    assert L.fathom_scan(*with_(0, MIS)) == F.ERR_ALIGN


def test_scan_rejects_plane_spans_past_31_bit_offsets(L):
    """A pair's plane rows (D x 4 x L words) must span less than 2^31 bytes,
    the range of the scan's buffer offsets: at D = 128 that is L < 2^19."""
    base = [A, A, 1, 128, 4096, 0, A, A, A, A, 4, A, None]

    def scan(n, cap, D=128, planes=A):
        b = list(base)
        b[0], b[3], b[4], b[5] = planes, D, n, cap
        return L.fathom_scan(*b)
    # capacity index: 2^19 + 1 blocks per row, few tokens
    assert scan(4096, (1 << 19) + 1) == F.ERR_UNSUPPORTED
    assert scan(4096, 1 << 19) == F.ERR_UNSUPPORTED        # exactly 2^31 bytes
    # dense index of 2^25 + 64 tokens: 2^19 + 1 blocks
    assert scan((1 << 25) + 64, 0) == F.ERR_UNSUPPORTED
    # the same row length at half the channels fits: the next check (a
    # misaligned planes pointer) is the one that fails
    assert scan((1 << 25) + 64, 0, D=64, planes=MIS) == F.ERR_ALIGN
    assert scan(4096, (1 << 19) - 1, planes=MIS) == F.ERR_ALIGN
    # fused path: the same check before the workspace is looked at
    ws = L.fathom_scan_topk_workspace_bytes(1, 4, 4096, 64)
    fused = [A, A, 1, 128, 4096, (1 << 19) + 1, A, A, A, A, 4, 64, A, None, A, A, A, ws, None]
    assert L.fathom_scan_topk(*fused) == F.ERR_UNSUPPORTED
    assert L.fathom_scan_topk_stage(2, *fused) == F.ERR_UNSUPPORTED


def test_pack_range_validation(L):
    # keys, dtype, P, tok0, m, D, rot, planes, scales, nb_cap, stream
    base = [A, 0, 2, 128, 10, 128, None, A, A, 4, None]

    def with_(i, v):
        b = list(base)
        b[i] = v
        return b
    assert L.fathom_pack_range(*with_(0, None)) == F.ERR_ARG
    assert L.fathom_pack_range(*with_(1, 5)) == F.ERR_ARG
    assert L.fathom_pack_range(*with_(3, 100)) == F.ERR_ARG   # not a block boundary
    assert L.fathom_pack_range(*with_(3, -64)) == F.ERR_ARG
    assert L.fathom_pack_range(*with_(4, 0)) == F.ERR_SHAPE
    assert L.fathom_pack_range(*with_(4, 200)) == F.ERR_SHAPE  # past the 4-block capacity
    assert L.fathom_pack_range(*with_(9, 2)) == F.ERR_SHAPE
    assert L.fathom_pack_range(*with_(5, 129)) == F.ERR_SHAPE
    assert L.fathom_pack_range(*with_(7, MIS)) == F.ERR_ALIGN


def test_topk_validation(L):
    ws = L.fathom_topk_workspace_bytes(2, 4, 4096, 64)
    assert ws > 0
    assert L.fathom_topk_workspace_bytes(2, 4, 4096, 5000) == 0
    ok = lambda **kw: [kw.get("s", A), 2, kw.get("G", 4), kw.get("n", 4096), kw.get("k", 64), A, None,
                       A, A, kw.get("ws", A), kw.get("wsb", ws), None]
    assert L.fathom_topk(*ok(s=None)) == F.ERR_ARG
    assert L.fathom_topk(*ok(k=0)) == F.ERR_ARG
    assert L.fathom_topk(*ok(k=4097, n=10000)) == F.ERR_UNSUPPORTED
    assert L.fathom_topk(*ok(G=8, k=4096)) == F.ERR_UNSUPPORTED
    assert L.fathom_topk(*ok(k=5000)) == F.ERR_ARG
    assert L.fathom_topk(*ok(wsb=ws - 1)) == F.ERR_WORKSPACE
    assert L.fathom_topk(*ok(ws=None)) == F.ERR_WORKSPACE
    assert L.fathom_topk(*ok(s=MIS)) == F.ERR_ALIGN
    assert L.fathom_topk(*ok(G=0)) == F.ERR_SHAPE


def test_workspace_scales_with_sample_stride(L):
    # 1M tokens, 288 pairs x 4 heads, k = 512: candidate lists stay well below
    # the 4.8 GB a full score copy would need
    b = L.fathom_topk_workspace_bytes(288, 4, 1 << 20, 512)
    assert 0 < b < 1 << 30


def test_gather_validation(L):
    args = lambda **kw: [kw.get("t", A), kw.get("rows", 1000), kw.get("rb", 512), kw.get("ps", 1000), 2,
                         A, A, kw.get("cap", 64), kw.get("out", A), None]
    assert L.fathom_gather_rows(*args(t=None)) == F.ERR_ARG
    assert L.fathom_gather_rows(*args(out=None)) == F.ERR_ARG
    assert L.fathom_gather_rows(*args(rb=500)) == F.ERR_SHAPE
    assert L.fathom_gather_rows(*args(rb=0)) == F.ERR_SHAPE
    assert L.fathom_gather_rows(*args(cap=0)) == F.ERR_SHAPE
    assert L.fathom_gather_rows(*args(ps=999)) == F.ERR_SHAPE
    ok = args()
    ok[4] = 65536
    assert L.fathom_gather_rows(*ok) == F.ERR_SHAPE
    assert L.fathom_gather_rows(*args(t=MIS)) == F.ERR_ALIGN


def test_calib_validation(L):
    ws = L.fathom_calib_workspace_bytes(2, 5000, 128)
    assert ws > 0
    assert L.fathom_calib_workspace_bytes(0, 5000, 128) == 0
    assert L.fathom_calib_workspace_bytes(2, 5000, 129) == 0
    args = lambda **kw: [kw.get("k", A), kw.get("dt", 1), 2, kw.get("m", 5000), 128, kw.get("cov", A),
                         kw.get("var", A), kw.get("ws", A), kw.get("wsb", ws), None]
    assert L.fathom_calib_covariance(*args(k=None)) == F.ERR_ARG
    assert L.fathom_calib_covariance(*args(cov=None, var=None)) == F.ERR_ARG
    assert L.fathom_calib_covariance(*args(dt=3)) == F.ERR_ARG
    assert L.fathom_calib_covariance(*args(m=0)) == F.ERR_SHAPE
    assert L.fathom_calib_covariance(*args(wsb=ws - 1)) == F.ERR_WORKSPACE
    assert L.fathom_calib_covariance(*args(ws=None)) == F.ERR_WORKSPACE
    assert L.fathom_calib_covariance(*args(cov=MIS)) == F.ERR_ALIGN
    assert L.fathom_calib_basis(None, 2, 128, A, A, None) == F.ERR_ARG
    assert L.fathom_calib_basis(A, 2, 129, A, A, None) == F.ERR_SHAPE
    assert L.fathom_calib_basis(A, 0, 128, A, A, None) == F.ERR_SHAPE
    assert L.fathom_calib_basis(MIS, 2, 128, A, A, None) == F.ERR_ALIGN


def test_binding_refuses_host_tensors():
    """The binding hands the library raw addresses; a host tensor has none
    the GPU can read, so it is refused before any call."""
    import torch

    with pytest.raises(ValueError, match="device memory"):
        F._ptr(torch.zeros(4))
    assert F._ptr(None) is None
    assert F._ptr(4096).value == 4096


def test_fused_workspace_is_bounded(L):
    """The fused scan + top-k keeps a bounded number of full score rows for
    the heads its sampled threshold misjudges (16 pairs' worth at most), so
    at 1M tokens x 288 pairs its workspace stays below 1 GiB, a fifth of a
    full score copy; it grows with the pairs only through the candidate
    lists."""
    npad = 1 << 20
    full = 288 * 4 * npad * 4
    b288 = L.fathom_scan_topk_workspace_bytes(288, 4, npad, 512)
    assert 0 < b288 < 1 << 30 and b288 < full // 5
    b8 = L.fathom_scan_topk_workspace_bytes(8, 4, npad, 512)
    b16 = L.fathom_scan_topk_workspace_bytes(16, 4, npad, 512)
    b32 = L.fathom_scan_topk_workspace_bytes(32, 4, npad, 512)
    assert b8 >= 8 * 4 * npad * 4  # fewer pairs than rows: one row per pair
    assert b32 - b16 < 16 * 4 * npad * 4  # beyond 16 pairs no more rows


def test_noalloc_rejects_calls_beyond_its_scratch(L):
    """fathom_scan_topk_noalloc checks its arguments and the size of the
    call against its fixed scratch before any HIP call."""
    args = lambda **kw: [A, A, kw.get("P", 8), 128, kw.get("n", 4096), 0, A, A, A, A, 4, kw.get("k", 64),
                         A, None, A, A, None]
    assert L.fathom_scan_topk_noalloc(*args(P=288, n=1 << 20, k=512)) == F.ERR_WORKSPACE
    assert L.fathom_scan_topk_noalloc(*args(P=8, n=1 << 23, k=512)) == F.ERR_WORKSPACE
    assert L.fathom_scan_topk_noalloc(*args(k=0)) == F.ERR_ARG
    assert L.fathom_scan_topk_noalloc(*args(P=0)) == F.ERR_SHAPE
    a = args()
    a[0] = None
    assert L.fathom_scan_topk_noalloc(*a) == F.ERR_ARG


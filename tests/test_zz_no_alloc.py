"""The allocation-free fused entry point, fathom_scan_topk_noalloc (its
workspace is the library's fixed per-GPU scratch), against fathom_scan_topk
with a workspace of its own: the same kernels run, so every output must be
the same bits.  Calls follow one another on the one scratch: a large one, a
smaller one after it (the scratch keeps the first call's contents), one
whose every pair needs the repair rows, and one over an index in host
memory (the staged sample in the scratch)."""
import numpy as np
import pytest
import torch

from tests.gpu_util import dev, need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def F():
    need_gpu()
    from sparse_attention_key_amd import fathom

    fathom.lib()
    return fathom


def _inputs(F, P, n, G, D, budget, seed, zero_q=False):
    g = np.random.default_rng(seed)
    x = np.stack([(g.standard_normal((n, D)) * np.exp(0.6 * g.standard_normal(D))).astype(np.float32)
                  for _ in range(P)])
    q = (g.standard_normal((P, G, D)) * np.exp(g.standard_normal((P, 1, D)))).astype(np.float32)
    if zero_q:
        q[:] = 0.0  # every score ties: every candidate list overflows
    s2 = np.exp(g.standard_normal((P, D))).astype(np.float32)
    planes, scales = F.pack(dev(x))
    pl = F.plan(dev(q), dev(s2), budget, 0)
    return planes, scales, pl


def _check_same(F, planes, scales, n, pl, k):
    ref = F.scan_topk(planes, scales, n, pl, k)
    got = F.TopkOut(pl.P, pl.G, n, k, "cuda", workspace=False)
    assert got.ws is None
    for t in (got.idx, got.union, got.union_len):
        t.fill_(-7)
    got.val.fill_(float("nan"))
    F.scan_topk_noalloc_into(planes, scales, n, pl, got)
    torch.cuda.synchronize()
    assert torch.equal(got.idx, ref.idx)
    assert torch.equal(got.val.view(torch.int32), ref.val.view(torch.int32))
    assert torch.equal(got.union_len, ref.union_len)
    assert torch.equal(got.union, ref.union)


def test_noalloc_matches_the_workspace_entry_point_on_consecutive_calls(F):
    for P, n, G, D, k, seed in ((8, 200000 + 37, 4, 128, 512, 1), (3, 5000 + 7, 2, 64, 64, 2)):
        say("no-alloc fused scan + top-k", P, n, G, D, k)
        planes, scales, pl = _inputs(F, P, n, G, D, 48, seed)
        _check_same(F, planes, scales, n, pl, k)


def test_noalloc_repairs_failed_pairs_in_the_scratch(F):
    say("no-alloc fused scan + top-k, every pair repaired")
    planes, scales, pl = _inputs(F, 20, 3000 + 5, 4, 128, 48, 3, zero_q=True)
    _check_same(F, planes, scales, 3000 + 5, pl, 100)
    planes, scales, pl = _inputs(F, 5, 777, 4, 128, 48, 4)
    _check_same(F, planes, scales, 777, pl, 50)


def test_noalloc_reads_a_host_index_once(F):
    """An index in mapped pinned host memory takes the staged sample (the
    sample's scores kept in the scratch, the filter skipping the sampled
    runs); the outputs equal the workspace entry point's on the same index
    in device memory."""
    from sparse_attention_key_amd.hostmem import PinnedHost

    P, n, k = 4, 300000 + 13, 512
    say("no-alloc fused scan + top-k, index in host memory", P, n, k)
    planes, scales, pl = _inputs(F, P, n, 4, 128, 48, 5)
    ph = PinnedHost(planes.numel() * 8)
    sh = PinnedHost(scales.numel() * 2)
    st = torch.cuda.current_stream()
    ph.copy_from_device(0, planes.data_ptr(), planes.numel() * 8, st)
    sh.copy_from_device(0, scales.data_ptr(), scales.numel() * 2, st)
    torch.cuda.synchronize()
    ref = F.scan_topk(planes, scales, n, pl, k)
    got = F.TopkOut(P, 4, n, k, "cuda", workspace=False)
    F.scan_topk_noalloc_into(ph.dev, sh.dev, n, pl, got)
    torch.cuda.synchronize()
    assert torch.equal(got.idx, ref.idx)
    assert torch.equal(got.val.view(torch.int32), ref.val.view(torch.int32))
    assert torch.equal(got.union_len, ref.union_len) and torch.equal(got.union, ref.union)
    ph.free()
    sh.free()


def test_noalloc_rejects_a_call_larger_than_the_scratch(F):
    say("no-alloc fused scan + top-k, too large")
    pl = F.Plan(288, 4, 128, "cuda")
    out = F.TopkOut(288, 4, 1 << 20, 512, "cuda", workspace=False)
    with pytest.raises(F.FathomError) as e:
        F.scan_topk_noalloc_into(4096, 4096, 1 << 20, pl, out)
    assert e.value.status == F.ERR_WORKSPACE

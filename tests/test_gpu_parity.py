"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Bit-exact: pack (planes, scales), plan (depths, level, active list, q_used),
scores (the fixed-point contract), top-k indices and values, union.  Scores are also checked against
the float64 definition: |s - s_def| <= 1e-5 |s_def| + 1e-6 ||q_h||_1 max scale.
Inputs all come from the seeded generators in workloads/ or numpy.
"""
import zlib

import numpy as np
import pytest
import torch

import workloads as wl
from tests.gpu_util import assert_selection_valid, bf16_dev, dev, need_gpu, say, score_tol, u16, u64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def F():
    need_gpu()
    from sparse_attention_key_amd import fathom

    fathom.lib()
    return fathom


def _np_keys(case):
    g = np.random.default_rng(zlib.crc32(case.encode()))
    if case == "tiny_f32":
        return wl.keys_host(wl.WORKLOADS["tiny"], 0), "f32"
    if case == "ragged_bf16":
        return wl.keys_host(wl.WORKLOADS["qwen32k"], 3, n=4096 + 37), "bf16"
    if case == "n1":
        return g.standard_normal((1, 128)).astype(np.float32), "f32"
    if case == "n63":
        return g.standard_normal((63, 128)).astype(np.float32), "f32"
    if case == "n65_bf16":
        return wl.to_bf16_exact(g.standard_normal((65, 128)).astype(np.float32) * 7), "bf16"
    if case == "d64":
        return g.standard_normal((1000, 64)).astype(np.float32), "f32"
    if case == "d96":
        return g.standard_normal((777, 96)).astype(np.float32), "f32"
    if case == "d100_bf16":  # D not a multiple of 8: the pack's one-element staging path
        return wl.to_bf16_exact(g.standard_normal((333, 100)).astype(np.float32) * 3), "bf16"
    if case == "boundaries":
        x = g.standard_normal((64 * 6, 128)).astype(np.float32)
        sc = np.abs(x).reshape(6, 64, 128).max(1).astype(np.float16).astype(np.float32)
        cells = g.integers(-8, 8, x.shape).astype(np.float32)
        x = (cells * np.repeat(sc, 64, 0) / np.float32(8)).astype(np.float32)
        x[::64] = np.repeat(sc, 1, 0)  # put the max back in every block
        x[1::64] = -np.repeat(sc, 1, 0)
        x[:, :16] = np.nextafter(x[:, :16], np.float32(np.inf))
        x[:, 16:32] = np.nextafter(x[:, 16:32], np.float32(-np.inf))
        x[:, 32:40] = 0.0
        x[:, 40:48] *= np.float32(1e-6)
        x[:64, 48] = np.float32(70000.0)  # saturating scale
        return x, "f32"
    raise KeyError(case)


PACK_CASES = ["tiny_f32", "ragged_bf16", "n1", "n63", "n65_bf16", "d64", "d96", "d100_bf16", "boundaries"]


@pytest.mark.parametrize("case", PACK_CASES)
def test_pack_bit_exact(F, orc, case):
    x, dt = _np_keys(case)
    say("pack", case, x.shape, dt)
    keys = (bf16_dev(x) if dt == "bf16" else dev(x))[None]
    planes, scales = F.pack(keys)
    rp, rs = orc.pack(x)
    assert np.array_equal(u16(scales)[0], rs)
    assert np.array_equal(u64(planes)[0], rp)


def test_pack_multi_pair_and_rotation(F, orc):
    g = np.random.default_rng(7)
    xs = [g.standard_normal((300, 128)).astype(np.float32) * np.exp(g.standard_normal(128)).astype(np.float32)
          for _ in range(3)]
    rots = [orc.calib.klt_basis(g.standard_normal((2000, 128)) @ g.standard_normal((128, 128)))[0]
            for _ in range(3)]
    say("pack multi-pair + rotation")
    keys = dev(np.stack(xs))
    planes, scales = F.pack(keys)
    planes_r, scales_r = F.pack(keys, rot=dev(np.stack(rots)))
    for p in range(3):
        rp, rs = orc.pack(xs[p])
        assert np.array_equal(u64(planes)[p], rp) and np.array_equal(u16(scales)[p], rs)
        rp, rs = orc.pack(xs[p], rot=rots[p])
        assert np.array_equal(u64(planes_r)[p], rp) and np.array_equal(u16(scales_r)[p], rs)


def _plan_inputs(P, G, D, seed):
    g = np.random.default_rng(seed)
    q = g.standard_normal((P, G, D)).astype(np.float32)
    q *= np.exp(g.standard_normal((P, 1, D)) * 1.5).astype(np.float32)
    s2 = np.exp(g.standard_normal((P, D)) * 2).astype(np.float32)
    s2[0, :3] = 0.0
    if P > 2:
        s2[1] = s2[1, 0]  # all weights driven by q only
        q[2, :, :D // 2] = q[2, :, D - D // 2:]  # repeated weights (ties at the level)
    return q, s2


PLAN_CASES = [(0, b) for b in (0, 1, 7, 32, 48, 68, 92, 136, 300, 511, 512)] + \
             [(1, r) for r in (0, 16, 32, 128)] + [(2, d) for d in (0, 1, 2, 4)]


@pytest.mark.parametrize("mode,budget", PLAN_CASES)
def test_plan_bit_exact(F, orc, mode, budget):
    P, G, D = 12, 4, 128
    q, s2 = _plan_inputs(P, G, D, 100 + budget)
    say("plan", mode, budget)
    pl = F.plan(dev(q), dev(s2), budget, mode)
    depth = pl.depth.cpu().numpy()
    act = pl.active.cpu().numpy()
    na = pl.n_active.cpu().numpy()
    th = pl.theta.cpu().numpy()
    qu = pl.q_used.cpu().numpy()
    for p in range(P):
        rd, rth, rq = orc.plan(q[p], s2[p], budget, mode)
        assert np.array_equal(depth[p], rd), p
        assert th[p].view(np.uint32) == np.float32(rth).view(np.uint32)
        assert np.array_equal(qu[p].view(np.uint32), rq.view(np.uint32))
        nz = np.nonzero(rd)[0]
        assert na[p] == nz.size
        assert np.array_equal(act[p, :nz.size], nz) and np.all(act[p, nz.size:] == -1)


@pytest.mark.parametrize("G,D", [(4, 128), (1, 128), (8, 64), (3, 96)])
def test_plan_rotated_and_shapes(F, orc, G, D):
    P = 5
    q, s2 = _plan_inputs(P, G, D, 7 * G + D)
    g = np.random.default_rng(G * D)
    rot = np.stack([np.linalg.qr(g.standard_normal((D, D)))[0] for _ in range(P)]).astype(np.float32)
    say("plan rotated", G, D)
    pl = F.plan(dev(q), dev(s2), 48, 0, rot=dev(rot))
    for p in range(P):
        rd, rth, rq = orc.plan(q[p], s2[p], 48, 0, rot=rot[p])
        assert np.array_equal(pl.depth.cpu().numpy()[p], rd)
        assert np.array_equal(pl.q_used.cpu().numpy()[p].view(np.uint32), rq.view(np.uint32))


@pytest.mark.parametrize("G,D,mode,budget", [(1, 1, 0, 2), (2, 16, 0, 20), (5, 33, 0, 40), (8, 65, 0, 100),
                                             (3, 127, 1, 16), (7, 100, 2, 3), (8, 128, 0, 48)])
def test_plan_odd_shapes_bit_exact(F, orc, G, D, mode, budget):
    """Plans at channel counts that leave lanes without a channel (D below
    64, between 64 and 128) and head counts from 1 to 8, in the stored basis:
    depths, level, scaled queries and active list equal the oracle's bit for
    bit."""
    P = 6
    q, s2 = _plan_inputs(P, G, D, 31 * G + D)
    say("plan odd shape", G, D, mode, budget)
    pl = F.plan(dev(q), dev(s2), budget, mode)
    depth, act, na = pl.depth.cpu().numpy(), pl.active.cpu().numpy(), pl.n_active.cpu().numpy()
    th, qu = pl.theta.cpu().numpy(), pl.q_used.cpu().numpy()
    for p in range(P):
        rd, rth, rq = orc.plan(q[p], s2[p], budget, mode)
        assert np.array_equal(depth[p], rd), p
        assert th[p].view(np.uint32) == np.float32(rth).view(np.uint32)
        assert np.array_equal(qu[p].view(np.uint32), rq.view(np.uint32))
        nz = np.nonzero(rd)[0]
        assert na[p] == nz.size
        assert np.array_equal(act[p, :nz.size], nz) and np.all(act[p, nz.size:] == -1)


SCAN_CASES = [  # (n, D, G, mode, budget)
    (4096, 128, 4, 0, 48), (4096 + 37, 128, 4, 0, 48), (1, 128, 4, 0, 48), (700, 128, 4, 0, 512),
    (700, 128, 4, 0, 0), (2000, 128, 4, 1, 32), (2000, 128, 4, 2, 2), (1500, 64, 8, 0, 92),
    (999, 96, 1, 0, 136), (3333, 128, 7, 0, 17),
]


@pytest.mark.parametrize("n,D,G,mode,budget", SCAN_CASES)
def test_scan_bit_exact_and_within_tolerance(F, orc, n, D, G, mode, budget):
    P = 2
    g = np.random.default_rng(n + D + G + budget)
    x = [(g.standard_normal((n, D)) * np.exp(g.standard_normal(D))).astype(np.float32) for _ in range(P)]
    q, s2 = _plan_inputs(P, G, D, n)
    say("scan", n, D, G, mode, budget)
    planes, scales = F.pack(dev(np.stack(x)))
    pl = F.plan(dev(q), dev(s2), budget, mode)
    scores = F.scan(planes, scales, n, pl).cpu().numpy()
    for p in range(P):
        rp, rs = orc.pack(x[p])
        rd, _, rq = orc.plan(q[p], s2[p], budget, mode)
        ref = orc.scores(rp, rs, n, rd, rq)
        assert np.array_equal(scores[p].view(np.uint32), ref.view(np.uint32))
        d64 = orc.ref64.scores_def(rp, rs, n, rd, rq)
        assert np.all(np.abs(scores[p][:, :n] - d64) <= score_tol(d64, rq, rs))


@pytest.mark.parametrize("mode,budget", [(1, 32), (1, 56), (2, 4)])
def test_scan_reads_the_last_plane_row_at_an_odd_block_count(F, orc, mode, budget):
    """Plans whose slot groups are equally deep take the scan form that reads
    two blocks per 16-byte load; the pair's very last plane row (channel
    D-1, plane 3) ends at an odd block count, so that load is moved back 8
    bytes.  Channel D-1 is made the most energetic so the fixed plans read
    it at depth 4 (A = 32, 56 and 128: all three slot-group widths)."""
    P, G, D, n = 2, 4, 128, 64 * 8 + 9  # 9 blocks
    g = np.random.default_rng(mode * 100 + budget)
    x = [(g.standard_normal((n, D)) * np.exp(0.5 * g.standard_normal(D))).astype(np.float32) for _ in range(P)]
    q, s2 = _plan_inputs(P, G, D, 321 + budget)
    q[:, :, D - 1] = 40.0
    say("scan, last plane row at an odd block count", mode, budget)
    planes, scales = F.pack(dev(np.stack(x)))
    pl = F.plan(dev(q), dev(s2), budget, mode)
    assert int(pl.depth[0, D - 1]) == 4 and int(pl.depth[1, D - 1]) == 4
    scores = F.scan(planes, scales, n, pl).cpu().numpy()
    out = F.scan_topk(planes, scales, n, pl, 64)
    for p in range(P):
        rp, rs = orc.pack(x[p])
        ref = orc.step(rp, rs, n, q[p], s2[p], budget, 64, mode=mode)
        assert np.array_equal(scores[p].view(np.uint32), ref["scores"].view(np.uint32))
        assert np.array_equal(out.idx[p].cpu().numpy(), ref["topk"])
        assert np.array_equal(out.union[p].cpu().numpy(), ref["union"])


def _topk_check(F, orc, s, n, k):
    P, G, _ = s.shape
    out = F.topk(dev(s), n, k)
    idx = out.idx.cpu().numpy()
    val = out.val.cpu().numpy()
    un = out.union.cpu().numpy()
    ul = out.union_len.cpu().numpy()
    for p in range(P):
        refs = []
        for h in range(G):
            ri, rv = orc.topk(s[p, h], n, k)
            assert np.array_equal(idx[p, h], ri), (p, h)
            assert np.array_equal(val[p, h], rv)
            refs.append(ri)
        ru, rl = orc.union(np.stack(refs))
        assert ul[p] == rl and np.array_equal(un[p], ru)


TOPK_CASES = [  # (n, k, kind)
    (4096, 64, "normal"), (32768, 512, "normal"), (100000, 512, "ties"), (70, 70, "normal"),
    (1, 1, "normal"), (64 * 33 + 5, 200, "ties"), (20000, 4096, "normal"), (5000, 1, "ties"),
    (200000, 512, "allequal"), (131072, 2048, "normal"),
    # both selection forms at their boundary (k <= 2048: 8 register slots and
    # a 2048-entry winner buffer), with thousands of tied candidates
    (150000, 2000, "ties"), (300000, 2048, "ties"), (60000, 2049, "ties"),
    (200000, 2000, "coarse"),  # ~13k candidates tie at the cut: past the register slots
]


@pytest.mark.parametrize("n,k,kind", TOPK_CASES)
def test_topk_union_bit_exact(F, orc, n, k, kind):
    P, G = 2, 4
    npad = (n + 63) // 64 * 64
    g = np.random.default_rng(n + k)
    s = g.standard_normal((P, G, npad)).astype(np.float32)
    if kind == "ties":
        s = np.round(s * 3).astype(np.float32)
        s[..., ::5] = -0.0
    if kind == "coarse":  # five or so distinct values: thousands tie at the k-th
        s = np.round(s).astype(np.float32)
    if kind == "allequal":  # every score tied: candidates overflow -> dense path
        s[:] = 1.5
    s[..., n:] = -np.inf
    say("topk", n, k, kind)
    _topk_check(F, orc, s, n, k)


def _run_pipeline(F, planes, scales, n, q, s2, budget, k, mode=0, rot=None):
    pl = F.plan(q, s2, budget, mode, rot=rot)
    scores = F.scan(planes, scales, n, pl)
    out = F.topk(scores, n, k)
    return pl, scores, out


def _compare_pair(orc, p, x, q, s2, budget, k, n, pl, scores, out, mode=0, rot=None, keys_rot=None):
    rp, rs = orc.pack(x, rot=keys_rot)
    ref = orc.step(rp, rs, n, q, s2, budget, k, mode=mode, rot=rot)
    assert np.array_equal(pl.depth[p].cpu().numpy(), ref["depth"])
    assert np.array_equal(scores[p].cpu().numpy().view(np.uint32), ref["scores"].view(np.uint32))
    assert np.array_equal(out.idx[p].cpu().numpy(), ref["topk"])
    assert out.union_len[p].item() == ref["union_len"]
    assert np.array_equal(out.union[p].cpu().numpy(), ref["union"])
    assert_selection_valid(orc, rp, rs, n, ref["depth"], ref["q_used"], out.idx[p].cpu().numpy())
    return rp, rs


def test_end_to_end_tiny(F, orc):
    w = wl.WORKLOADS["tiny"]
    x = wl.keys_host(w, 0)
    q = wl.queries(w, 0)
    s2 = orc.calib.channel_variance(wl.calibration_sample(w, 0))
    say("end-to-end tiny")
    planes, scales = F.pack(dev(x)[None])
    pl, scores, out = _run_pipeline(F, planes, scales, w.n, dev(q)[None], dev(s2)[None], w.budget, w.k)
    _compare_pair(orc, 0, x, q, s2, w.budget, w.k, w.n, pl, scores, out)
    pos = wl.planted_positions(w, 0)
    for h in range(w.G):
        assert set(pos[h]) <= set(out.idx[0, h].cpu().numpy())


def test_end_to_end_qwen32k(F, orc):
    w = wl.WORKLOADS["qwen32k"]
    xs = [wl.keys_host(w, p) for p in range(w.P)]
    qs = np.stack([wl.queries(w, p) for p in range(w.P)])
    s2 = np.stack([orc.calib.channel_variance(wl.calibration_sample(w, p)) for p in range(w.P)])
    say("end-to-end qwen32k")
    planes, scales = F.pack(bf16_dev(np.stack(xs)))
    pl, scores, out = _run_pipeline(F, planes, scales, w.n, dev(qs), dev(s2), w.budget, w.k)
    for p in range(w.P):
        _compare_pair(orc, p, xs[p], qs[p], s2[p], w.budget, w.k, w.n, pl, scores, out)


def test_end_to_end_rotated_small(F, orc):
    w = wl.WORKLOADS["host1m_klt"]
    n = 5000
    P = 2
    xs = [wl.keys_host(w, p, n=n) for p in range(P)]
    qs = np.stack([wl.queries(w, p) for p in range(P)])
    rots, lams = zip(*[orc.calib.klt_basis(wl.calibration_sample(w, p)) for p in range(P)])
    rot = np.stack(rots)
    lam = np.stack(lams)
    say("end-to-end rotated small")
    planes, scales = F.pack(bf16_dev(np.stack(xs)), rot=dev(rot))
    pl, scores, out = _run_pipeline(F, planes, scales, n, dev(qs), dev(lam), w.budget, w.k, rot=dev(rot))
    for p in range(P):
        _compare_pair(orc, p, xs[p], qs[p], lam[p], w.budget, w.k, n, pl, scores, out,
                      rot=rot[p], keys_rot=rot[p])


FUSED_CASES = [  # (workload-ish, n, D, G, budget, k, mode)
    ("rand", 4096, 128, 4, 48, 64, 0), ("rand", 32768 + 17, 128, 4, 48, 512, 0),
    ("rand", 700, 128, 4, 48, 512, 0), ("rand", 5000, 64, 8, 92, 256, 0),
    ("rand", 20000, 128, 4, 0, 300, 0),      # every score 0: ties overflow -> repair path
    ("rand", 9000, 128, 2, 32, 1, 1), ("rand", 100, 128, 4, 2, 100, 2), ("rand", 1, 128, 4, 48, 1, 0),
    ("rand", 3000, 100, 4, 40, 128, 0),   # D not a multiple of 8
]


@pytest.mark.parametrize("kind,n,D,G,budget,k,mode", FUSED_CASES)
def test_fused_scan_topk_bit_exact(F, orc, kind, n, D, G, budget, k, mode):
    P = 3
    g = np.random.default_rng(n * 7 + budget + k)
    x = [(g.standard_normal((n, D)) * np.exp(0.7 * g.standard_normal(D))).astype(np.float32) for _ in range(P)]
    q, s2 = _plan_inputs(P, G, D, n + 1)
    say("fused scan+top-k", n, D, G, budget, k, mode)
    planes, scales = F.pack(dev(np.stack(x)))
    pl = F.plan(dev(q), dev(s2), budget, mode)
    out = F.scan_topk(planes, scales, n, pl, k)
    staged = F.TopkOut(P, G, n, k, "cuda", fused=True)
    for stage in (1, 2, 3):
        F.scan_topk_stage(stage, planes, scales, n, pl, staged)
    idx = out.idx.cpu().numpy()
    val = out.val.cpu().numpy()
    assert np.array_equal(idx, staged.idx.cpu().numpy())
    assert np.array_equal(out.union.cpu().numpy(), staged.union.cpu().numpy())
    for p in range(P):
        rp, rs = orc.pack(x[p])
        ref = orc.step(rp, rs, n, q[p], s2[p], budget, k, mode=mode)
        assert np.array_equal(idx[p], ref["topk"]), p
        for h in range(G):
            assert np.array_equal(val[p, h], ref["scores"][h][ref["topk"][h]])
        assert int(out.union_len[p]) == ref["union_len"]
        assert np.array_equal(out.union[p].cpu().numpy(), ref["union"])
        assert_selection_valid(orc, rp, rs, n, ref["depth"], ref["q_used"], idx[p])


def _random_fused_cases(count=24, seed=20261203):
    """Seeded random shapes for the fused path: n from 1 to 20,000 (ragged
    blocks), D from 16 to 128 (not only multiples of 8 or 32), G from 1 to 8,
    every plan mode with a budget across its whole range, k from 1 to
    min(n, 2048, 16384 / G)."""
    g = np.random.default_rng(seed)
    cases = []
    for i in range(count):
        n = int(g.integers(1, 20001)) if i % 3 else int(g.integers(1, 400))
        D = int(g.choice([16, 33, 48, 64, 100, 127, 128]))
        G = int(g.integers(1, 9))
        mode = int(g.choice([0, 0, 0, 1, 2]))
        budget = int(g.integers(0, 4 * D + 1)) if mode == 0 else int(g.integers(0, D + 1)) if mode == 1 \
            else int(g.integers(0, 5))
        k = int(g.integers(1, min(n, 2048, 16384 // G) + 1))
        cases.append((n, D, G, budget, k, mode))
    return cases


@pytest.mark.parametrize("n,D,G,budget,k,mode", _random_fused_cases())
def test_fused_random_shapes_bit_exact(F, orc, n, D, G, budget, k, mode):
    P = 2
    g = np.random.default_rng(n * 131 + D * 7 + G + budget * 3 + k)
    x = [(g.standard_normal((n, D)) * np.exp(0.7 * g.standard_normal(D))).astype(np.float32) for _ in range(P)]
    q, s2 = _plan_inputs(P, G, D, n + 3)
    say("fused random shape", n, D, G, budget, k, mode)
    planes, scales = F.pack(dev(np.stack(x)))
    pl = F.plan(dev(q), dev(s2), budget, mode)
    out = F.scan_topk(planes, scales, n, pl, k)
    idx = out.idx.cpu().numpy()
    for p in range(P):
        rp, rs = orc.pack(x[p])
        ref = orc.step(rp, rs, n, q[p], s2[p], budget, k, mode=mode)
        assert np.array_equal(idx[p], ref["topk"]), p
        assert int(out.union_len[p]) == ref["union_len"]
        assert np.array_equal(out.union[p].cpu().numpy(), ref["union"])


def test_fused_repair_with_more_failed_pairs_than_rows(F, orc):
    """Every third pair has an all-zero query, so all its scores tie and its
    candidate lists overflow; with 37 pairs that is 13 failed pairs, and
    with 20 of them (every pair) more failures than the 16 repair rows, so
    each repair workgroup rescans several pairs in turn.  Every pair's
    top-k and union must equal the oracle's bit for bit."""
    G, D, n, k, budget = 4, 128, 3000 + 5, 100, 48
    for P, zero in ((37, lambda p: p % 3 == 0), (20, lambda p: True)):
        g = np.random.default_rng(P)
        x = [(g.standard_normal((n, D)) * np.exp(0.5 * g.standard_normal(D))).astype(np.float32)
             for _ in range(P)]
        q, s2 = _plan_inputs(P, G, D, 1000 + P)
        for p in range(P):
            if zero(p):
                q[p] = 0.0
        say("fused repair, failed pairs:", sum(zero(p) for p in range(P)), "of", P)
        planes, scales = F.pack(dev(np.stack(x)))
        pl = F.plan(dev(q), dev(s2), budget, 0)
        out = F.scan_topk(planes, scales, n, pl, k)
        idx = out.idx.cpu().numpy()
        val = out.val.cpu().numpy()
        for p in range(P):
            rp, rs = orc.pack(x[p])
            ref = orc.step(rp, rs, n, q[p], s2[p], budget, k)
            assert np.array_equal(idx[p], ref["topk"]), p
            for h in range(G):
                assert np.array_equal(val[p, h], ref["scores"][h][ref["topk"][h]])
            assert int(out.union_len[p]) == ref["union_len"]
            assert np.array_equal(out.union[p].cpu().numpy(), ref["union"]), p


def _sample_stride(n, k):
    """One run of 32 blocks in every s runs is sampled for the fused
    threshold: s is the largest power of two with (2s)^2 4k <= n kept."""
    nb = (n + 63) // 64
    s = 1
    while (2 * s) ** 2 * 4 * k <= n and 2 * s <= nb:
        s *= 2
    return s


def test_fused_fallback_when_the_sample_threshold_passes_too_few(F, orc):
    """Keys planted in the first sampled run score far above everything else,
    so the sample threshold (the ceil(2k/s)-th sampled score) leaves fewer
    than k candidates for those heads.  Stage 3 must then select over every
    score of the head: the result still equals the oracle bit for bit."""
    P, G, D, n, k, budget = 2, 4, 128, 65536 + 300, 64, 48
    g = np.random.default_rng(20261203)
    scale = np.exp(0.7 * g.standard_normal(D)).astype(np.float32)
    x = [(g.standard_normal((n, D)) * scale).astype(np.float32) for _ in range(P)]
    q, s2 = _plan_inputs(P, G, D, 77)
    rms = float(np.sqrt(np.mean(scale.astype(np.float64) ** 2)))
    for p in range(P):
        for h in range(G):
            qh = q[p, h].astype(np.float64)
            for i in range(12):  # distinct 16-token groups, all inside blocks 0..31
                tok = 40 * (12 * h + i) + 3
                x[p][tok] = (qh * (8.0 * rms / np.linalg.norm(qh))).astype(np.float32)
    s = _sample_stride(n, k)
    assert s > 1 and n < 128 * k * s  # token-level sample, one run in every s
    rank = -(-2 * k // s)
    say("fused fallback: planted sample winners", n, k, s)
    planes, scales = F.pack(dev(np.stack(x)))
    pl = F.plan(dev(q), dev(s2), budget, 0)
    out = F.scan_topk(planes, scales, n, pl, k)
    idx = out.idx.cpu().numpy()
    val = out.val.cpu().numpy()
    nb = (n + 63) // 64
    sampled = np.zeros(n, bool)
    for b0 in range(0, nb, 32 * s):
        sampled[b0 * 64:min(n, (b0 + 32) * 64)] = True
    short = 0
    for p in range(P):
        rp, rs = orc.pack(x[p])
        ref = orc.step(rp, rs, n, q[p], s2[p], budget, k)
        for h in range(G):
            sc = ref["scores"][h][:n]
            thr = np.sort(sc[sampled])[::-1][rank - 1]
            short += int((sc >= thr).sum() < k)
            assert np.array_equal(idx[p, h], ref["topk"][h]), (p, h)
            assert np.array_equal(val[p, h], sc[ref["topk"][h]])
        assert np.array_equal(out.union[p].cpu().numpy(), ref["union"])
    assert short == P * G  # every head needed the fallback


def test_fused_threshold_keeps_candidate_lists_in_range(F, orc):
    """On ordinary keys the sampled threshold (group-of-16 maxima of one run
    in every s, estimated from the top digit rows) must leave between k and
    the list capacity candidates for every head, so no head needs the full
    rescan: a wrong sample stage would still give exact results through the
    rescan, and only this check sees it.  The result must equal the
    materialised path's (scores stored, then selected)."""
    import torch

    P, G, D, n, k, budget = 2, 4, 128, 524288 + 77, 256, 48
    g = np.random.default_rng(4242)
    x = [(g.standard_normal((n, D)) * np.exp(0.7 * g.standard_normal(D))).astype(np.float32) for _ in range(P)]
    q, s2 = _plan_inputs(P, G, D, 4243)
    s = _sample_stride(n, k)
    assert n >= 128 * k * s and -(-2 * k // s) == 32  # group maxima; threshold at the 32nd
    say("fused threshold range", n, k, s)
    planes, scales = F.pack(dev(np.stack(x)))
    pl = F.plan(dev(q), dev(s2), budget, 0)
    out = F.TopkOut(P, G, n, k, pl.q_used.device, fused=True)
    F.scan_topk_stage(1, planes, scales, n, pl, out)
    F.scan_topk_stage(2, planes, scales, n, pl, out)
    m = P * G
    off = (m * 4 + 255) // 256 * 256  # candidate counts follow the thresholds
    counts = out.ws[off:off + 4 * m].view(torch.int32).cpu().numpy()
    cap = 8 * k * s + 1024
    assert (counts >= k).all() and (counts <= cap).all(), counts
    assert counts.mean() < 8 * k, counts  # about 2k expected
    F.scan_topk_stage(3, planes, scales, n, pl, out)
    ref = F.topk(F.scan(planes, scales, n, pl), n, k)
    assert np.array_equal(out.idx.cpu().numpy(), ref.idx.cpu().numpy())
    assert np.array_equal(out.union.cpu().numpy(), ref.union.cpu().numpy())


def test_host_resident_index_matches_device(F, orc):
    """The scan reads a mapped pinned host copy of the index over the host
    link and must give the same bits as from HBM (KLT-rotated storage)."""
    import torch

    from sparse_attention_key_amd.hostmem import PinnedHost

    w = wl.WORKLOADS["host1m_klt"]
    P, n = 2, 40000 + 11
    xs = [wl.keys_host(w, p, n=n) for p in range(P)]
    qs = np.stack([wl.queries(w, p) for p in range(P)])
    rots, lams = zip(*[orc.calib.klt_basis(wl.calibration_sample(w, p)) for p in range(P)])
    rot, lam = np.stack(rots), np.stack(lams)
    say("host-resident index", n)
    planes, scales = F.pack(bf16_dev(np.stack(xs)), rot=dev(rot))
    ph = PinnedHost(planes.numel() * 8)
    sh = PinnedHost(scales.numel() * 2)
    st = torch.cuda.current_stream()
    ph.copy_from_device(0, planes.data_ptr(), planes.numel() * 8, st)
    sh.copy_from_device(0, scales.data_ptr(), scales.numel() * 2, st)
    torch.cuda.synchronize()
    pl = F.plan(dev(qs), dev(lam), w.budget, 0, rot=dev(rot))
    ref = F.scan_topk(planes, scales, n, pl, w.k)
    got = F.scan_topk(ph.dev, sh.dev, n, pl, w.k)
    s_dev = F.scan(planes, scales, n, pl)
    s_host = F.scan(ph.dev, sh.dev, n, pl)
    torch.cuda.synchronize()
    assert torch.equal(s_dev, s_host)
    assert torch.equal(ref.idx, got.idx) and torch.equal(ref.union, got.union)
    for p in range(P):
        _compare_pair(orc, p, xs[p], qs[p], lam[p], w.budget, w.k, n, pl, s_host, got,
                      rot=rot[p], keys_rot=rot[p])
    ph.free()
    sh.free()


@pytest.mark.parametrize("k,mode,budget", [(64, 0, 48), (512, 0, 48), (512, 1, 32)])
def test_host_resident_staged_sample(F, orc, k, mode, budget):
    """Over the host link the sample stage keeps its scores and the filter
    skips the sampled runs (every index byte read once).  At n = 600,013 the
    sample is one run in 32 for k = 64 (group maxima set the threshold, the
    scores are stored beside them) and one run in 16 for k = 512 (every
    sampled score, which are also the stored ones).  The 136-bit fixed plan
    (mode 1, r = 32) takes the slot-shared scan form.  One call, the three
    stages called one by one, and the same step from HBM must all give the
    same winners, values and unions, equal to the oracle's."""
    import torch

    from sparse_attention_key_amd.hostmem import PinnedHost

    w = wl.WORKLOADS["host1m_klt"]
    P, n = 3, 600000 + 13
    s = _sample_stride(n, k)
    assert s == (32 if k == 64 else 16) and (n >= 128 * k * s) == (k == 64)
    xs = [wl.keys_host(w, p, n=n) for p in range(P)]
    qs = np.stack([wl.queries(w, p) for p in range(P)])
    rots, lams = zip(*[orc.calib.klt_basis(wl.calibration_sample(w, p)) for p in range(P)])
    rot, lam = np.stack(rots), np.stack(lams)
    say("host-resident staged sample", n, k, mode, budget)
    planes, scales = F.pack(bf16_dev(np.stack(xs)), rot=dev(rot))
    ph = PinnedHost(planes.numel() * 8)
    sh = PinnedHost(scales.numel() * 2)
    st = torch.cuda.current_stream()
    ph.copy_from_device(0, planes.data_ptr(), planes.numel() * 8, st)
    sh.copy_from_device(0, scales.data_ptr(), scales.numel() * 2, st)
    torch.cuda.synchronize()
    pl = F.plan(dev(qs), dev(lam), budget, mode, rot=dev(rot))
    ref = F.scan_topk(planes, scales, n, pl, k)
    got = F.scan_topk(ph.dev, sh.dev, n, pl, k)
    staged = F.TopkOut(P, w.G, n, k, pl.q_used.device, fused=True)
    for stage in (1, 2, 3):
        F.scan_topk_stage(stage, ph.dev, sh.dev, n, pl, staged)
    s_host = F.scan(ph.dev, sh.dev, n, pl)
    torch.cuda.synchronize()
    for o in (got, staged):
        assert torch.equal(ref.idx, o.idx) and torch.equal(ref.val, o.val)
        assert torch.equal(ref.union, o.union) and torch.equal(ref.union_len, o.union_len)
    _compare_pair(orc, 0, xs[0], qs[0], lam[0], budget, k, n, pl, s_host, got, mode=mode, rot=rot[0],
                  keys_rot=rot[0])
    ph.free()
    sh.free()


def test_host_resident_small_workspace_falls_back(F):
    """A workspace large enough for the device layout but not for the staged
    sample (here 40 pairs at 65,536 tokens, k = 64: the stored sample scores,
    one 512-block run per pair, take 20 MiB against the 16 MiB of repair rows
    they share memory with) still gives the same results over the host link,
    without the staging."""
    from sparse_attention_key_amd.hostmem import PinnedHost

    P, G, D, n, k = 40, 4, 128, 65536, 64
    g = np.random.default_rng(515)
    x = (g.standard_normal((P, n, D)) * np.exp(0.7 * g.standard_normal((P, 1, D)))).astype(np.float32)
    q, s2 = _plan_inputs(P, G, D, 516)
    say("host-resident index, workspace below the staged layout", P, n, k)
    planes, scales = F.pack(dev(x))
    del x
    ph = PinnedHost(planes.numel() * 8)
    sh = PinnedHost(scales.numel() * 2)
    st = torch.cuda.current_stream()
    ph.copy_from_device(0, planes.data_ptr(), planes.numel() * 8, st)
    sh.copy_from_device(0, scales.data_ptr(), scales.numel() * 2, st)
    torch.cuda.synchronize()
    pl = F.plan(dev(q), dev(s2), 48, 0)
    ref = F.scan_topk(planes, scales, n, pl, k)
    full = F.scan_topk_workspace_bytes(P, G, n, k)
    outs = []
    for ws_bytes in (full, full - (512 << 10)):
        o = F.TopkOut(P, G, n, k, pl.q_used.device, fused=True)
        o.ws = torch.empty(ws_bytes, dtype=torch.uint8, device=pl.q_used.device)
        F.scan_topk_into(ph.dev, sh.dev, n, pl, o)
        outs.append(o)
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(ref.idx, o.idx) and torch.equal(ref.val, o.val)
        assert torch.equal(ref.union, o.union) and torch.equal(ref.union_len, o.union_len)
    ph.free()
    sh.free()


@pytest.mark.parametrize("shared,host", [(False, False), (True, False), (False, True), (True, True)])
def test_gather_rows_bit_exact(F, orc, shared, host):
    """Winner-row fetch: union rows of every pair copied out of a K|V row
    table in HBM or in mapped pinned host memory."""
    import torch

    from sparse_attention_key_amd.hostmem import PinnedHost

    P, rows, row_bytes, cap = 3, 5000, 512, 700
    g = np.random.default_rng(11 + shared + 2 * host)
    shape = (rows, row_bytes // 2) if shared else (P, rows, row_bytes // 2)
    table = g.integers(0, 65536, shape, dtype=np.uint16)
    idx = np.full((P, cap), -1, np.int32)
    lens = np.array([0, 357, cap], np.int32)
    for p in range(P):
        idx[p, :lens[p]] = np.sort(g.choice(rows, lens[p], replace=False))
    idx[2, 5] = rows + 3  # an index outside the table is skipped
    say("gather", shared, host)
    tdev = torch.from_numpy(table.view(np.int16)).cuda()
    src = tdev
    ph = None
    if host:
        ph = PinnedHost(table.nbytes)
        ph.copy_from_device(0, tdev.data_ptr(), table.nbytes, torch.cuda.current_stream())
        torch.cuda.synchronize()
        src = ph.dev
    init = g.integers(0, 65536, (P, cap, row_bytes // 2), dtype=np.uint16)
    out = torch.from_numpy(init.view(np.int16)).cuda()
    F.gather_rows(src, rows, row_bytes, 0 if shared else rows, dev(idx), dev(lens), out)
    got = out.cpu().numpy().view(np.uint16)
    ref = orc.gather_rows(table, idx, lens, init)
    assert np.array_equal(got, ref)
    if ph is not None:
        ph.free()


# ------------------------------------------------------- appends (pack_range)

SENTINEL = -0x0123456789ABCDF  # marks index words no call may touch


def _cap_index(P, D, cap, device="cuda"):
    planes = torch.full((P, D, 4, cap), SENTINEL, dtype=torch.int64, device=device)
    scales = torch.full((P, D, cap), -1, dtype=torch.int16, device=device)
    return planes, scales


def test_append_token_by_token_matches_full_pack(F, orc):
    P, D, n0, n1, cap = 3, 128, 600, 1000, 20  # 1000 tokens fill 16 blocks of a 20-block capacity
    g = np.random.default_rng(41)
    x = [wl.to_bf16_exact((g.standard_normal((n1, D)) * np.exp(0.8 * g.standard_normal(D))).astype(np.float32))
         for _ in range(P)]
    xd = bf16_dev(np.stack(x))
    say("append", P, n0, "->", n1, "capacity", cap)
    planes, scales = _cap_index(P, D, cap)
    F.pack_range(xd[:, :n0].contiguous(), 0, planes, scales)
    for t in range(n0, n1):  # token t arrives: repack its block from that block's raw keys
        tok0 = (t // 64) * 64
        F.pack_range(xd[:, tok0:t + 1].contiguous(), tok0, planes, scales)
    torch.cuda.synchronize()
    nb = (n1 + 63) // 64
    got_p, got_s = u64(planes), u16(scales)
    for p in range(P):
        rp, rs = orc.pack(x[p])
        assert np.array_equal(got_p[p][:, :, :nb], rp), p
        assert np.array_equal(got_s[p][:, :nb], rs), p
    assert np.all(planes[:, :, :, nb:].cpu().numpy() == SENTINEL)
    assert np.all(scales[:, :, nb:].cpu().numpy() == -1)


def test_pack_range_offset_and_rotation(F, orc):
    P, D, n, cap = 2, 128, 700, 16
    g = np.random.default_rng(42)
    x = [g.standard_normal((n, D)).astype(np.float32) * 3 for _ in range(P)]
    rot = np.stack([np.linalg.qr(g.standard_normal((D, D)))[0].astype(np.float32) for _ in range(P)])
    say("pack_range offset 128, 300 tokens, rotated")
    planes, scales = _cap_index(P, D, cap)
    F.pack_range(dev(np.stack(x))[:, 128:428].contiguous(), 128, planes, scales, rot=dev(rot))
    torch.cuda.synchronize()
    got_p, got_s = u64(planes), u16(scales)
    for p in range(P):
        # blocks 2..6 hold tokens 128..427; block 6 is partial (tokens 384..427)
        rp, rs = orc.pack(x[p][128:428], rot=rot[p])
        assert np.array_equal(got_p[p][:, :, 2:7], rp), p
        assert np.array_equal(got_s[p][:, 2:7], rs), p
    assert np.all(planes[:, :, :, :2].cpu().numpy() == SENTINEL)
    assert np.all(planes[:, :, :, 7:].cpu().numpy() == SENTINEL)


def test_scan_topk_on_capacity_index(F, orc):
    P, D, G, n, cap, budget, k = 3, 128, 4, 5000, 100, 48, 256
    g = np.random.default_rng(43)
    x = [(g.standard_normal((n, D)) * np.exp(0.7 * g.standard_normal(D))).astype(np.float32) for _ in range(P)]
    q, s2 = _plan_inputs(P, G, D, n + 3)
    say("scan+top-k on a capacity index", n, cap)
    xd = dev(np.stack(x))
    planes, scales = _cap_index(P, D, cap)
    F.pack_range(xd, 0, planes, scales)
    dense_p, dense_s = F.pack(xd)
    pl = F.plan(dev(q), dev(s2), budget)
    out = F.scan_topk(planes, scales, n, pl, k)
    ref_out = F.scan_topk(dense_p, dense_s, n, pl, k)
    scores = F.scan(planes, scales, n, pl)
    ref_scores = F.scan(dense_p, dense_s, n, pl)
    assert torch.equal(out.idx, ref_out.idx) and torch.equal(out.union, ref_out.union)
    assert torch.equal(scores.view(torch.int32), ref_scores.view(torch.int32))
    for p in range(P):
        rp, rs = orc.pack(x[p])
        ref = orc.step(rp, rs, n, q[p], s2[p], budget, k)
        assert np.array_equal(out.idx[p].cpu().numpy(), ref["topk"]), p
        assert np.array_equal(out.union[p].cpu().numpy(), ref["union"]), p


def test_binding_refuses_strided_tensors(F):
    """A transposed view has the right shape but not the row-major layout
    the entry points read: the binding refuses it instead of passing its
    storage through (a transposed rotation would silently give another
    plan)."""
    import torch

    rot = torch.eye(64, device="cuda") + torch.arange(4096, device="cuda").reshape(64, 64) / 4096
    q = torch.ones((1, 2, 64), device="cuda")
    s2 = torch.ones((1, 64), device="cuda")
    with pytest.raises(ValueError, match="not contiguous"):
        F.plan(q, s2, 16, 0, rot=rot.t().unsqueeze(0))
    F.plan(q, s2, 16, 0, rot=rot.t().contiguous().unsqueeze(0))


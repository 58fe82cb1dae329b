"""Pins of the CPU oracle against what the pages and mathematics fix.

Nothing here retypes the oracle's formulas: each check compares the oracle
with a library routine, a brute-force search, a closed form, an invariant or
exact rational arithmetic.  Sources: yeyulingfeng.com write-up of Fathom
(arXiv 2609.17652), sections "方法一" (bit planes), "方法二" (reverse
water-filling), "基座选择" (basis), and the paotong.dev bit-plane figure.
"""
import numpy as np
import pytest

from tests.exact_fp import fma32, mul32
import workloads as wl


# --------------------------------------------------------------- binary16

def test_f16_conversion_matches_numpy(orc):
    g = np.random.default_rng(1)
    vals = np.concatenate([
        g.standard_normal(3000) * 10.0 ** g.integers(-9, 5, 3000),
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e-8, 2.0 ** -24, 2.0 ** -25,
                  2.0 ** -25 * 1.5, 3 * 2.0 ** -26, 6.1e-5, 2.0 ** -14, 1.0 + 2.0 ** -11,
                  1.0 + 3 * 2.0 ** -11, 2047.0, 2049.0, 4097.0])]).astype(np.float32)
    for v in vals:
        ref = int(np.float32(v).astype(np.float16).view(np.uint16))
        assert orc.f32_to_f16_bits(v) == ref, v
        if not np.isinf(np.float16(v)):
            assert orc.f16_bits_to_f32(ref) == np.float32(np.float16(v)), v


# ------------------------------------------------------------------- pack

def _adversarial_block(g, D=128):
    """64 tokens x D channels with values on cell boundaries, at +-max, zero
    blocks and maxima that round up or down when stored in fp16."""
    x = g.standard_normal((64, D)).astype(np.float32)
    for j in range(D):
        kind = j % 8
        m = np.float32(abs(x[:, j]).max())
        if kind == 0:  # exact cell boundaries k * scale/8 of the stored scale
            sc = np.float32(np.float16(m))
            ks = g.integers(-8, 8, 64)
            x[:, j] = (ks * (sc / np.float32(8))).astype(np.float32)
            x[0, j] = sc
        elif kind == 1:  # block max exactly at +m and -m
            x[0, j], x[1, j] = m, -m
        elif kind == 2:  # all zero
            x[:, j] = 0.0
        elif kind == 3:  # max that fp16 rounds up (scale > m)
            x[0, j] = np.float32(1.0 + 2.0 ** -12 + 2.0 ** -20)
            x[1:, j] = np.clip(x[1:, j], -1, 1)
        elif kind == 4:  # max that fp16 rounds down (scale < m): codes clamp
            x[0, j] = np.float32(1.0 + 2.0 ** -12 - 2.0 ** -20)
            x[1:, j] = np.clip(x[1:, j], -1, 1)
        elif kind == 5:  # tiny magnitudes (fp16 subnormal scales)
            x[:, j] *= np.float32(1e-6)
        elif kind == 6:  # values one ulp either side of boundaries
            sc = np.float32(np.float16(m))
            b = (g.integers(-7, 8, 64) * (sc / np.float32(8))).astype(np.float32)
            x[:, j] = np.where(g.random(64) < 0.5, np.nextafter(b, np.float32(np.inf)),
                               np.nextafter(b, np.float32(-np.inf)))
            x[0, j] = sc
    return x


def test_pack_matches_floor_definition(orc):
    g = np.random.default_rng(2)
    x = np.concatenate([_adversarial_block(g), g.standard_normal((200, 128)).astype(np.float32) * 3])
    n = x.shape[0]  # 264: ragged last block
    planes, scales = orc.pack(x)
    nb = (n + 63) // 64
    assert planes.shape == (128, 4, nb) and scales.shape == (128, nb)
    # scale = fp16 RNE of the block max over valid tokens (numpy conversion)
    for b in range(nb):
        m = np.abs(x[64 * b:64 * (b + 1)]).max(axis=0)
        assert np.array_equal(scales[:, b], m.astype(np.float16).view(np.uint16))
    codes = orc.ref64.decode_codes(planes, n)
    ref = orc.ref64.pack_codes_def(x, orc.ref64.f16_bits_to_f64(scales))
    assert np.array_equal(codes, ref)
    # padding tokens carry code 8
    allc = orc.ref64.decode_codes(planes, nb * 64)
    assert np.all(allc[:, n:] == 8)


def test_pack_invariants(orc):
    g = np.random.default_rng(3)
    x = g.standard_normal((640, 128)).astype(np.float32) * np.exp(g.standard_normal(128)).astype(np.float32)
    planes, scales = orc.pack(x)
    codes = orc.ref64.decode_codes(planes, 640)
    sc = orc.ref64.f16_bits_to_f64(scales)[:, np.arange(640) // 64]
    # the sign plane is x >= 0 (code 8 is the cell starting at zero)
    assert np.array_equal(codes >> 3, (x.T >= 0).astype(np.int64))
    # full-depth reconstruction error is at most half a cell where |x| <= scale
    k4 = orc.ref64.dequant(codes, 4, sc)
    inside = np.abs(x.T) <= sc
    assert np.all(np.abs(x.T - k4)[inside] <= sc[inside] / 16 + 1e-30)


def test_index_footprint_68_bytes():
    # bit-plane section: 64 plane bytes + one fp16 per 64 tokens per channel
    D = 128
    plane_bytes = D * 4 * 8 / 64
    scale_bytes = D * 2 / 64
    assert plane_bytes + scale_bytes == 68.0


# --------------------------------------------------------- prefix decode

@pytest.mark.parametrize("t", [1, 2, 3, 4])
def test_prefix_equals_direct_requantisation(orc, t):
    g = np.random.default_rng(10 + t)
    x = np.concatenate([_adversarial_block(g), g.uniform(-1, 1, (128, 128)).astype(np.float32)])
    planes, scales = orc.pack(x)
    n = x.shape[0]
    codes = orc.ref64.decode_codes(planes, n)
    sc = orc.ref64.f16_bits_to_f64(scales)[:, np.arange(n) // 64]
    inside = (np.abs(x.T) <= sc) & (sc > 0)
    direct = orc.ref64.requant_direct(x.T, sc, t)
    assert np.array_equal(orc.ref64.prefix_code(codes, t)[inside], direct[inside])
    # C prefix reader agrees with the numpy decode
    for (j, i) in [(0, 0), (5, 63), (17, 64), (127, n - 1), (64, 100)]:
        assert orc.lib().orc_prefix_code(planes.ctypes.data, planes.shape[2], j, i, t) == codes[j, i] >> (4 - t)


def test_dequant_values_and_full_depth(orc):
    # t = 1 reads only the sign: +-scale/2 = +-4 cells
    for sb in [0x3C00, 0x4248, 0x0001, 0x7BFF]:
        s = orc.f16_bits_to_f32(sb)
        assert orc.dequant(1, 1, sb) == np.float32(s / 2)
        assert orc.dequant(0, 1, sb) == np.float32(-s / 2)
        assert orc.dequant(5, 0, sb) == 0.0
        for t in range(1, 5):
            for c in range(2 ** t):
                ref = orc.ref64.dequant(c, t, s)
                assert orc.dequant(c, t, sb) == ref  # exact
        # t = 4 is the original 4-bit cell midpoint (c - 8 + 1/2) * scale/8
        for c in range(16):
            assert orc.dequant(c, 4, sb) == (c - 7.5) * s / 8


def test_error_variance_quarters_per_plane(orc):
    # each extra plane divides the error variance by 4 (method two)
    g = np.random.default_rng(20)
    x = g.uniform(-1, 1, (64 * 2000, 1)).astype(np.float32)
    x[::64] = 1.0  # block max exactly 1 -> scale 1
    planes, scales = orc.pack(x)
    codes = orc.ref64.decode_codes(planes, x.shape[0])[0]
    sc = orc.ref64.f16_bits_to_f64(scales)[0, np.arange(x.shape[0]) // 64]
    mse = [np.mean((x[:, 0] - orc.ref64.dequant(orc.ref64.prefix_code(codes, t), t, sc)) ** 2)
           for t in range(1, 5)]
    for t in range(3):
        assert 3.8 < mse[t] / mse[t + 1] < 4.2
    assert abs(mse[3] / ((2.0 / 16) ** 2 / 12) - 1) < 0.05


# ------------------------------------------------------------------- plan

def test_plan_matches_exhaustive_search(orc):
    g = np.random.default_rng(30)
    cases = 0
    for D in (1, 2, 3, 4, 5):
        for rep in range(6):
            w = (np.exp(g.standard_normal(D) * 2.5)).astype(np.float32)
            if rep == 5:
                w[0] = 0.0
            for B in range(0, 4 * D + 2):
                theta = orc.water_level(w, B)
                t = np.array([orc.depth_at(v, theta) for v in w])
                best, args = orc.ref64.plan_bruteforce(w, B)
                assert t.sum() <= B
                assert orc.ref64.objective(w, t) == pytest.approx(best, rel=1e-12, abs=0)
                if len(args) == 1:
                    assert tuple(t) == args[0]
                cases += 1
    assert cases > 200


def test_water_level_equals_bitpattern_bisection(orc):
    g = np.random.default_rng(31)
    for rep in range(40):
        D = 128
        w = (np.exp(g.standard_normal(D) * 2.0) * 10.0 ** g.integers(-20, 20)).astype(np.float32)
        w[g.integers(0, D, 10)] = 0.0
        if rep % 7 == 0:
            w[:64] = w[64:]  # heavy ties
        if rep % 11 == 0:
            w[:5] = np.float32(1e-42)  # subnormal weights
        for B in (0, 1, 17, 48, 92, 136, 300, 512):
            th = orc.water_level(w, B)
            assert np.float32(th) == orc.ref64.water_level_bisect(w, B)
            t = orc.ref64.fp32_depths(w, np.float32(th))
            assert t.sum() <= B
            assert np.all(t[w == 0] == 0)
            assert np.all(t[w <= th] == 0)  # channels below the level are skipped
            if th > 0:  # the next-lower level overflows the budget
                below = np.nextafter(np.float32(th), np.float32(0))
                assert orc.ref64.fp32_depths(w, below).sum() > B
            else:
                assert np.all(t[w > 0] == 4)


def test_water_level_log_bisection_close(orc):
    g = np.random.default_rng(32)
    for _ in range(10):
        w = np.exp(g.standard_normal(128) * 2).astype(np.float32)
        th = orc.water_level(w, 48)
        lg = orc.ref64.water_level_log_bisect(w, 48)
        assert abs(lg / th - 1) < 1e-6 or orc.ref64.fp32_depths(w, np.float32(lg)).sum() <= 48


def test_depths_monotone_in_theta(orc):
    g = np.random.default_rng(33)
    w = np.exp(g.standard_normal(64) * 3).astype(np.float32)
    thetas = np.sort(np.exp(g.standard_normal(200) * 4)).astype(np.float32)
    prev = None
    for th in thetas:
        t = np.array([orc.depth_at(v, th) for v in w])
        if prev is not None:
            assert np.all(t <= prev)
        prev = t


def test_importance_uses_variance_and_query_energy(orc):
    # multiplying one channel's variance by 4 (or its query by 2 in every head)
    # moves it exactly one plane deeper at a fixed water level
    g = np.random.default_rng(34)
    q = g.standard_normal((4, 128)).astype(np.float32)
    s2 = np.exp(g.standard_normal(128)).astype(np.float32)
    w = orc.importance(q, s2)
    th = np.float32(np.sort(w)[64]) * np.float32(0.37)
    t0 = orc.ref64.fp32_depths(w, th)
    j = int(np.argmax((t0 > 0) & (t0 < 4)))
    s2b = s2.copy()
    s2b[j] *= 4
    qb = q.copy()
    qb[:, j] *= 2
    assert orc.ref64.fp32_depths(orc.importance(q, s2b), th)[j] == t0[j] + 1
    assert orc.ref64.fp32_depths(orc.importance(qb, s2), th)[j] == t0[j] + 1
    # exact value on tiny inputs: fp32 fma chain over heads, then one product
    for j in range(3):
        sq = np.float32(0)
        for h in range(4):
            sq = fma32(q[h, j], q[h, j], sq)
        assert w[j] == mul32(s2[j], sq)
    # a zero-variance channel is never read
    s2[7] = 0.0
    d, theta, _ = orc.plan(q, s2, 48)
    assert d[7] == 0


def test_plan_budget_extremes(orc):
    g = np.random.default_rng(35)
    q = g.standard_normal((4, 128)).astype(np.float32)
    s2 = np.exp(g.standard_normal(128)).astype(np.float32)
    d, th, _ = orc.plan(q, s2, 0)
    assert d.sum() == 0
    d, th, _ = orc.plan(q, s2, 512)
    assert np.all(d == 4) and th == 0.0
    for B in (32, 48, 68, 92, 136):
        d, th, _ = orc.plan(q, s2, B)
        assert d.sum() == B  # continuous random weights: no ties at the level


def test_fixed_topr_plan(orc):
    # 136-bit baseline: the 32 channels of largest group query energy at 4 planes
    g = np.random.default_rng(36)
    q = g.standard_normal((4, 128)).astype(np.float32)
    q[:, 10] = q[:, 11]  # a tie, broken toward the lower channel
    s2 = np.ones(128, np.float32)
    d, th, _ = orc.plan(q, s2, 32, mode=orc.PLAN_TOPR)
    energy = (q.astype(np.float64) ** 2).sum(0)
    order = np.lexsort((np.arange(128), -energy))
    assert set(np.nonzero(d)[0]) == set(order[:32])
    assert np.all(d[d > 0] == 4) and d.sum() == 128
    d, _, _ = orc.plan(q, s2, 2, mode=orc.PLAN_UNIFORM)
    assert np.all(d == 2)


def test_rotated_query(orc):
    g = np.random.default_rng(37)
    a = g.standard_normal((128, 128))
    U = np.linalg.qr(a)[0].astype(np.float32)
    q = g.standard_normal((4, 128)).astype(np.float32)
    k = g.standard_normal(128).astype(np.float32)
    qu = orc.query_used(q, U)
    ref = q.astype(np.float64) @ U.astype(np.float64)
    assert np.allclose(qu, ref, rtol=0, atol=1e-5)
    # rotation preserves dot products: (U^T q) . (U^T k) = q . k
    ku = (k.astype(np.float64) @ U.astype(np.float64))
    assert np.allclose(qu.astype(np.float64) @ ku, q.astype(np.float64) @ k, atol=1e-4)
    # fp32 fma chain over ascending d, checked exactly on the first outputs
    for j in range(2):
        acc = np.float32(0)
        for d in range(128):
            acc = fma32(U[d, j], q[0, d], acc)
        assert qu[0, j] == acc


# ------------------------------------------------------------------ scores

def _rand_index(orc, n, seed, D=128):
    g = np.random.default_rng(seed)
    x = (g.standard_normal((n, D)) * np.exp(0.5 * g.standard_normal(D))).astype(np.float32)
    planes, scales = orc.pack(x)
    q = g.standard_normal((4, D)).astype(np.float32)
    return x, planes, scales, q


def test_full_budget_is_full_4bit_dot(orc):
    n = 200
    x, planes, scales, q = _rand_index(orc, n, 40)
    depth = np.full(128, 4, np.uint8)
    s32 = orc.scores(planes, scales, n, depth, q)
    codes = orc.ref64.decode_codes(planes, n)
    sc = orc.ref64.f16_bits_to_f64(scales)[:, np.arange(n) // 64]
    k4 = (codes - 7.5) * sc / 8
    ref = q.astype(np.float64) @ k4
    assert np.all(np.isneginf(s32[:, n:]))
    tol = 1e-5 * np.abs(ref) + 1e-6 * np.abs(q).sum(1, keepdims=True) * sc.max()
    assert np.all(np.abs(s32[:, :n] - ref) <= tol)
    assert np.allclose(orc.scores_f64(planes, scales, n, depth, q), ref, rtol=1e-12, atol=1e-12)


def test_single_channel_single_plane_by_hand(orc):
    n = 64
    x = np.zeros((n, 128), np.float32)
    x[:, 3] = np.linspace(-2, 2, n).astype(np.float32)
    planes, scales = orc.pack(x)
    q = np.zeros((4, 128), np.float32)
    q[:, 3] = [1.0, -2.0, 0.5, 3.0]
    depth = np.zeros(128, np.uint8)
    depth[3] = 1
    s = orc.scores(planes, scales, n, depth, q)
    half = np.float32(orc.f16_bits_to_f32(scales[3, 0]) / 2)  # +-4 cells
    sign = np.where(x[:, 3] >= 0, 1.0, -1.0)
    assert np.array_equal(s[:, :n], (q[:, 3:4] * sign[None, :] * half).astype(np.float32))


def _def_and_bound(orc, planes, scales, n, depth, q):
    """float64 definition and the contract's stated error bound."""
    ref = orc.ref64.scores_def(planes, scales, n, depth, q)
    return ref, orc.ref64.contract_bound(planes, scales, n, depth, q, s_def=ref)


def test_fixed_point_scores_within_their_bound(orc):
    # the exact-integer contract differs from the real dot product only by
    # the coefficient truncation (bounded above) and one final rounding
    for seed, B, mag in ((41, 48, 1.0), (44, 136, 1.0), (45, 512, 1.0), (46, 7, 1.0), (50, 48, 1e-3)):
        n = 300
        x, planes, scales, q = _rand_index(orc, n, seed)
        if mag != 1.0:  # small keys: block scales far below 1 (binary16 exponent field ~ 5)
            planes, scales = orc.pack(x * np.float32(mag))
        s2 = np.exp(np.random.default_rng(seed).standard_normal(128)).astype(np.float32)
        depth, _, qu = orc.plan(q, s2, B)
        s = orc.scores(planes, scales, n, depth, qu)[:, :n].astype(np.float64)
        ref, bound = _def_and_bound(orc, planes, scales, n, depth, qu)
        assert np.all(np.abs(s - ref) <= bound)


def test_fixed_point_exact_when_representable(orc):
    # power-of-two queries and scales with a short mantissa make every
    # coefficient an exact integer: the score is the real dot product
    # rounded once (here exactly representable)
    n = 128
    g = np.random.default_rng(47)
    scales_pow = np.exp2(g.integers(-3, 4, 128)).astype(np.float32)
    x = (g.standard_normal((n, 128)) * scales_pow).astype(np.float32)
    planes, scales = orc.pack(x)
    scales = (scales & np.uint16(0xFE00)).astype(np.uint16)  # 2 mantissa bits left
    q = (np.exp2(g.integers(-4, 3, (4, 128))) * g.choice([-1, 1], (4, 128))).astype(np.float32)
    depth = g.integers(0, 5, 128).astype(np.uint8)
    s = orc.scores(planes, scales, n, depth, q)[:, :n].astype(np.float64)
    ref = orc.ref64.scores_def(planes, scales, n, depth, q)
    assert np.array_equal(s, ref.astype(np.float32).astype(np.float64))


def test_fixed_point_scale_invariance_and_block_locality(orc):
    n = 256
    x, planes, scales, q = _rand_index(orc, n, 48)
    depth = np.random.default_rng(49).integers(0, 5, 128).astype(np.uint8)
    s = orc.scores(planes, scales, n, depth, q)
    # a power-of-two query scale moves sigma and nothing else
    s8 = orc.scores(planes, scales, n, depth, q * np.float32(8))
    assert np.array_equal(s8[:, :n], (s[:, :n] * np.float32(8)))
    # block 2's scales do not enter the scores of blocks 0, 1 and 3
    sc2 = scales.copy()
    sc2[:, 2] = (sc2[:, 2].astype(np.int32) + 1024).astype(np.uint16)  # one binade up
    s2 = orc.scores(planes, sc2, n, depth, q)
    keep = np.r_[0:128, 192:256]
    assert np.array_equal(s2[:, keep], s[:, keep])
    assert not np.array_equal(s2[:, 128:192], s[:, 128:192])


def test_scores_within_tolerance_of_definition(orc):
    n = 1000
    x, planes, scales, q = _rand_index(orc, n, 42)
    s2 = np.exp(np.random.default_rng(43).standard_normal(128)).astype(np.float32)
    depth, theta, qu = orc.plan(q, s2, 48)
    s32 = orc.scores(planes, scales, n, depth, qu)[:, :n]
    ref = orc.ref64.scores_def(planes, scales, n, depth, qu)
    smax = orc.ref64.f16_bits_to_f64(scales).max()
    tol = 1e-5 * np.abs(ref) + 1e-6 * np.abs(qu).sum(1, keepdims=True) * smax
    assert np.all(np.abs(s32 - ref) <= tol)


def _selection_cases(orc):
    """(planes, scales, n, q, s2, budget, k) cases: random keys with wide
    channel scales at several budgets and k, and the tiny workload."""
    import workloads as wl

    cases = []
    for seed, n, B, k in ((60, 3000, 48, 64), (61, 3000, 7, 512), (62, 2500, 136, 1), (63, 4097, 512, 300),
                          (64, 3000, 32, 64)):
        x, planes, scales, q = _rand_index(orc, n, seed)
        s2 = np.exp(np.random.default_rng(seed + 1).standard_normal(128)).astype(np.float32)
        cases.append((planes, scales, n, q, s2, B, k))
    w = wl.WORKLOADS["tiny"]
    planes, scales = orc.pack(wl.keys_host(w, 0))
    s2 = orc.calib.channel_variance(wl.calibration_sample(w, 0))
    cases.append((planes, scales, w.n, wl.queries(w, 0), s2, w.budget, w.k))
    return cases


def test_contract_topk_is_a_valid_topk_of_the_definition(orc):
    # The selected sets are exact under the fixed-point contract; against the
    # plain float64 definition (the query times the prefix-dequantised keys)
    # they must be a top-k that the contract's stated error bound allows, and
    # exactly the definition's top-k wherever its k-th and (k+1)-th scores
    # are further apart than the bounds.
    forced = 0
    for planes, scales, n, q, s2, B, k in _selection_cases(orc):
        ref = orc.step(planes, scales, n, q, s2, B, k)
        s_def = orc.ref64.scores_def(planes, scales, n, ref["depth"], ref["q_used"])
        bnd = orc.ref64.contract_bound(planes, scales, n, ref["depth"], ref["q_used"], s_def=s_def)
        for h in range(q.shape[0]):
            assert orc.ref64.topk_valid(s_def[h], bnd[h], ref["topk"][h], n)
            order = orc.ref64.topk_def(s_def[h], n, n)
            win, rest = order[:k], order[k:]
            if rest.size == 0 or (s_def[h, win] - bnd[h, win]).min() > (s_def[h, rest] + bnd[h, rest]).max():
                forced += 1
                assert set(ref["topk"][h].tolist()) == set(win.tolist())
    assert forced >= 6  # the margin case is exercised, not only the band


def test_topk_validity_check_rejects_a_wrong_selection(orc):
    # the check has teeth: trading the weakest winner for the strongest loser
    # (far apart here) or repeating a token is not a valid top-k
    planes, scales, n, q, s2, B, k = _selection_cases(orc)[0]
    ref = orc.step(planes, scales, n, q, s2, B, k)
    s_def = orc.ref64.scores_def(planes, scales, n, ref["depth"], ref["q_used"])
    bnd = orc.ref64.contract_bound(planes, scales, n, ref["depth"], ref["q_used"], s_def=s_def)
    order = orc.ref64.topk_def(s_def[0], n, n)
    bad = order[:k].copy()
    bad[-1] = order[-1]  # the lowest-scoring token instead of the k-th
    assert not orc.ref64.topk_valid(s_def[0], bnd[0], bad, n)
    dup = order[:k].copy()
    dup[-1] = dup[0]
    assert not orc.ref64.topk_valid(s_def[0], bnd[0], dup, n)
    assert orc.ref64.topk_valid(s_def[0], bnd[0], order[:k], n)


# ------------------------------------------------------------------ top-k

def test_topk_matches_full_sort(orc):
    g = np.random.default_rng(50)
    for n, k, ties in [(100, 10, False), (1000, 64, True), (4096, 512, True), (70, 70, False)]:
        s = g.standard_normal(n).astype(np.float32)
        if ties:
            s = np.round(s * 4).astype(np.float32)  # many equal scores
            s[::7] = -0.0
            s[1::7] = 0.0
        idx, val = orc.topk(s, n, k)
        assert np.array_equal(idx, orc.ref64.topk_def(s, n, k))
        assert np.array_equal(val, s[idx])


def test_union_matches_numpy(orc):
    g = np.random.default_rng(51)
    idx = g.integers(0, 300, (4, 64)).astype(np.int32)
    for h in range(4):
        idx[h] = g.choice(300, 64, replace=False)
    u, ln = orc.union(idx)
    ref = np.union1d(idx.ravel(), [])
    assert ln == ref.size and np.array_equal(u[:ln], ref) and np.all(u[ln:] == -1)


def test_tiny_planted_keys_win(orc):
    # not from the pages: a sanity check of the whole chain on the tiny workload
    w = wl.WORKLOADS["tiny"]
    x = wl.keys_host(w, 0)
    q = wl.queries(w, 0)
    s2 = orc.calib.channel_variance(wl.calibration_sample(w, 0))
    planes, scales = orc.pack(x)
    out = orc.step(planes, scales, w.n, q, s2, w.budget, w.k)
    pos = wl.planted_positions(w, 0)
    for h in range(w.G):
        assert set(pos[h]) <= set(out["topk"][h])
    assert out["union_len"] <= w.G * w.k


def test_gather_rows_definition(orc):
    # identity indices return the table's leading rows; a shared table equals
    # the same table replicated per pair; rows past the length stay untouched
    g = np.random.default_rng(60)
    table = g.integers(0, 1000, (50, 4))
    idx = np.tile(np.arange(10, dtype=np.int32), (2, 1))
    lens = np.array([10, 4], np.int32)
    init = -np.ones((2, 10, 4), np.int64)
    out = orc.gather_rows(table, idx, lens, init)
    assert np.array_equal(out[0], table[:10])
    assert np.array_equal(out[1, :4], table[:4]) and np.all(out[1, 4:] == -1)
    rep = orc.gather_rows(np.stack([table, table]), idx, lens, init)
    assert np.array_equal(out, rep)


# ------------------------------------------------------------ calibration

def test_channel_variance_closed_form(orc):
    # every channel j takes the values mu_j + a_j and mu_j - a_j equally often:
    # centred population variance a_j^2 exactly, whatever the mean
    D = 16
    a = np.arange(1, D + 1, dtype=np.float64) * 0.25
    mu = np.linspace(-40.0, 40.0, D)
    x = np.concatenate([mu + a, mu - a, mu - a, mu + a])[None].reshape(4, D)
    v = orc.calib.channel_variance(x)
    assert np.array_equal(v, (a * a).astype(np.float32))


def test_klt_basis_recovers_a_constructed_covariance(orc):
    # rows +-sqrt(D) s_i q_i (i < D) have mean 0 and covariance Q diag(s^2) Q^T,
    # so the basis must be Q (up to signs) with eigenvalues s^2, descending
    D = 24
    g = np.random.default_rng(5)
    Q = np.linalg.qr(g.standard_normal((D, D)))[0]
    s = np.linspace(3.0, 0.1, D)
    rows = [sign * np.sqrt(D) * s[i] * Q[:, i] for i in range(D) for sign in (1.0, -1.0)]
    U, lam = orc.calib.klt_basis(np.array(rows))
    assert np.allclose(lam, s * s, rtol=1e-6)
    assert np.allclose(np.abs(np.sum(U * Q, axis=0)), 1.0, atol=1e-6)
    assert np.all(np.diff(lam) <= 0)

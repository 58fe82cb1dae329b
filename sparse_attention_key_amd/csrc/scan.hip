// Approximate scores of every key from the bit-plane index (yeyulingfeng.com
// write-up of Fathom: section "方法一" -- a t-plane prefix is the t-bit
// mid-rise quantiser; section "方法二" -- only the first t_j planes of each
// active channel are read, and the plan is shared by the G heads of a group
// so the index is read once for all of them; limitations section -- one
// shift-and-mask per extracted bit and G multiply-adds per element).
//
// Score contract: for token i and head h, s = 0 and for each active channel
// j in ascending order s = fma(q_hj, khat_ij, s), with khat_ij the exact
// dequantised prefix (2 c_t + 1 - 2^t) * 2^-t * scale.
//
// Mapping (gfx950, wave64).  A lane owns TOK consecutive tokens of one
// 64-token block (TOK = 32 for G <= 4, 16 for G <= 8, so that TOK * G = 128
// fp32 accumulators per lane); the 64/TOK lanes of a block sit 64/TOK*... apart
// so that one wavefront covers TOK consecutive blocks and every plane-word
// load is one contiguous 256 B (TOK=32) or 128 B (TOK=16) row segment.  Codes
// are extracted 4 (TOK=32) or 2 (TOK=16) tokens at a time: plane bit g of
// every byte is shifted to its place in the code and masked in one
// AND-OR, and v_cvt_f32_ubyte turns each byte into a float.  The next
// channel's plane words and scale are in flight while the current channel is
// accumulated.
//
// Output modes: STORE writes the scores; FILTER compares each score against
// the per-(pair, head) threshold and appends survivors as 64-bit
// (key, ~index) composites with one atomic per wavefront and head; LANEMAX
// writes, per lane and head, the largest score among the lane's tokens (over
// a sample of blocks: the input of the top-k threshold).
#include "common.h"

namespace fathom {
namespace {

constexpr int kScanThreads = 256;
constexpr int kRun = 32;  // sampled blocks come in runs of this many consecutive blocks

template <int TOK>
struct Words;
template <>
struct Words<32> {
    using T = uint32_t;
};
template <>
struct Words<16> {
    using T = uint16_t;
};

// Codes of the lane's TOK tokens for one channel.  Group g holds tokens g,
// g+8, g+16, g+24 (one per byte; two bytes when TOK = 16), and its code sits
// with the sign plane on bit m_g of the byte -- m_g = g for g >= 3, g + 4
// below -- and plane s on bit m_g - s.  Then plane s reaches every group
// with g >= 3 through one right shift by s and the others through one left
// shift by 4 - s, so a plane costs two shifts and one AND-OR per group; the
// byte of group g reads as c4 * 2^e_g (c4 = c_t * 2^(4-t), e_g = m_g - 3),
// and absent planes stay zero.
template <int TOK>
__device__ __forceinline__ void codes(const uint32_t (&w)[4], int t, uint32_t (&c)[8])
{
    constexpr uint32_t lanes = TOK == 32 ? 0x01010101u : 0x0101u;
#pragma unroll
    for (int g = 0; g < 8; ++g) c[g] = 0;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        if (s < t) {  // wavefront-uniform
            const uint32_t r = w[s] >> s, l = w[s] << (4 - s);
#pragma unroll
            for (int g = 0; g < 8; ++g)
                c[g] |= (g >= 3 ? r : l) & (lanes << ((g >= 3 ? g : g + 4) - s));
        }
    }
}

// power-of-two weight of group g's byte (see codes())
__host__ __device__ constexpr int group_exp(int g) { return g >= 3 ? g - 3 : g + 1; }

// acc += q_h * khat for the lane's tokens, with khat = byte * delta_e + c0 the
// exact dequantised prefix (delta_e = scale / 8 / 2^e for a byte weighted
// 2^e, c0 = (1 - 2^t) * 2^-t * scale).
template <int G, int TOK>
__device__ __forceinline__ void accumulate(const uint32_t (&c)[8], const float (&delta)[5], float c0,
                                           const float (&qv)[G], float (&acc)[G][TOK])
{
#pragma unroll
    for (int g = 0; g < 8; ++g) {
#pragma unroll
        for (int b = 0; b < TOK / 8; ++b) {
            const float cf = (float)((c[g] >> (8 * b)) & 0xFFu);
            const float kh = __builtin_fmaf(cf, delta[group_exp(g)], c0);  // exact
#pragma unroll
            for (int h = 0; h < G; ++h) acc[h][g + 8 * b] = __builtin_fmaf(qv[h], kh, acc[h][g + 8 * b]);
        }
    }
}

// Plane words and scale of one channel for one lane, loaded ahead of use.
// Loads are buffer loads: the channel's row base lives in an SGPR resource
// descriptor and the lane adds a small byte offset, so no per-lane 64-bit
// address arithmetic is spent.  Every channel issues exactly five loads --
// absent planes re-read plane 0, a cache hit that costs no HBM bytes -- so
// the number of loads in flight is static and the waits are exact.
template <class WT>
struct ChanWords {
    uint32_t w0, w1, w2, w3, sc;

    __device__ __forceinline__ void issue(const uint64_t* pplanes, const uint16_t* pscales,
                                          int64_t ldb, uint32_t loff, uint32_t soff, int jt_lds)
    {
        const int jt = __builtin_amdgcn_readfirstlane(jt_lds);
        const int j = jt & 0xFFFF, t = jt >> 16;
        const int row = (int)(ldb * 8);
        __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(pplanes + (size_t)j * 4 * ldb), (short)0, 4 * row, 0x00020000);
        __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(pscales + (size_t)j * ldb), (short)0, (int)(ldb * 2), 0x00020000);
        if (sizeof(WT) == 4) {
            w0 = __builtin_amdgcn_raw_buffer_load_b32(rp, loff, 0, 0);
            w1 = __builtin_amdgcn_raw_buffer_load_b32(rp, loff, t > 1 ? row : 0, 0);
            w2 = __builtin_amdgcn_raw_buffer_load_b32(rp, loff, t > 2 ? 2 * row : 0, 0);
            w3 = __builtin_amdgcn_raw_buffer_load_b32(rp, loff, t > 3 ? 3 * row : 0, 0);
        } else {
            w0 = __builtin_amdgcn_raw_buffer_load_b16(rp, loff, 0, 0);
            w1 = __builtin_amdgcn_raw_buffer_load_b16(rp, loff, t > 1 ? row : 0, 0);
            w2 = __builtin_amdgcn_raw_buffer_load_b16(rp, loff, t > 2 ? 2 * row : 0, 0);
            w3 = __builtin_amdgcn_raw_buffer_load_b16(rp, loff, t > 3 ? 3 * row : 0, 0);
        }
        sc = __builtin_amdgcn_raw_buffer_load_b16(rs, soff, 0, 0);
    }

    template <int G, int TOK>
    __device__ __forceinline__ void consume(int jt_lds, const float (&q)[G], float (&acc)[G][TOK]) const
    {
        const int t = __builtin_amdgcn_readfirstlane(jt_lds) >> 16;
        float qv[G];
#pragma unroll
        for (int h = 0; h < G; ++h) qv[h] = q[h];
        const uint32_t w[4] = {w0, w1, w2, w3};  // planes >= t are not read by codes()
        const float scf = (float)__builtin_bit_cast(_Float16, (uint16_t)sc);  // v_cvt_f32_f16, exact
        float delta[5];  // scale / 8 / 2^e, all exact
#pragma unroll
        for (int e = 0; e < 5; ++e) delta[e] = scf * (0.125f / (float)(1 << e));
        const float c0 = scf * __uint_as_float((uint32_t)(127 - t) << 23) * (float)(1 - (1 << t));
        uint32_t c[8];
        codes<TOK>(w, t, c);
        accumulate<G, TOK>(c, delta, c0, qv, acc);
    }
};

enum { kStore = 0, kFilter = 1, kLaneMax = 2 };

// One workgroup's tile of pair p.
template <int G, int TOK, int MODE>
__device__ __forceinline__ void scan_pair(const ScanArgs& a, const int p)
{
    constexpr int kParts = 64 / TOK;       // lanes per block
    constexpr int kBlocksPerWave = TOK;    // 64 / kParts
    using WT = typename Words<TOK>::T;
    __shared__ int s_jt[kMaxD];            // j | t << 16
    __shared__ float s_q[kMaxD][G];
    constexpr bool FILTER = MODE == kFilter;
    __shared__ __attribute__((aligned(16))) float s_stage[FILTER ? kScanThreads / kWave : 1][kWave][TOK + 4];
    __shared__ uint32_t s_wcount[kScanThreads / kWave][G];

    const int A = a.n_active[p];
    for (int e = threadIdx.x; e < A; e += kScanThreads) {
        const int j = a.active[(size_t)p * a.D + e];
        s_jt[e] = j | ((int)a.depth[(size_t)p * a.D + j] << 16);
#pragma unroll
        for (int h = 0; h < G; ++h) s_q[e][h] = a.q_used[((size_t)p * G + h) * a.D + j];
    }
    __syncthreads();

    const int lane = lane_id(), wave = threadIdx.x / kWave;
    const int part = lane / kBlocksPerWave;
    const int64_t lb = ((int64_t)blockIdx.x * (kScanThreads / kWave) + wave) * kBlocksPerWave +
                       (lane % kBlocksPerWave);
    const int64_t lb0 = lb - (lane % kBlocksPerWave);
    if (lb0 >= a.nlb) return;  // whole wavefront past the end
    // logical -> physical block: runs of kRun consecutive blocks, one run in
    // every `stride` (stride 1 is the identity)
    const int64_t phys = (lb / kRun) * kRun * a.stride + (lb % kRun);
    const bool live = lb < a.nlb && phys < a.nb;
    const int64_t blk = live ? phys : 0;
    const int64_t nb = a.ldb;  // row stride of the index, in blocks
    const uint64_t* pplanes = a.planes + (size_t)p * a.D * 4 * nb;  // uniform
    const uint16_t* pscales = a.scales + (size_t)p * a.D * nb;
    const uint32_t loff = (uint32_t)(blk * 8 + part * (int)sizeof(WT));
    const uint32_t soff = (uint32_t)(blk * 2);

    float acc[G][TOK];  // head-major: acc[h][i..i+3] are four consecutive registers
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int i = 0; i < TOK; ++i) acc[h][i] = 0.0f;

    // register sets in rotation, with no copies: while one channel is
    // accumulated the loads of the next two (one for G = 8, whose extra
    // accumulators leave no room for a third set) are in flight.  Indices
    // past the end re-issue the last channel: cache hits that nobody reads.
    if (A > 0) {
        const int last = A - 1;
        ChanWords<WT> X, Y;
        X.issue(pplanes, pscales, nb, loff, soff, s_jt[0]);
        if (G < 8) {
            ChanWords<WT> Z;
            Y.issue(pplanes, pscales, nb, loff, soff, s_jt[1 < A ? 1 : last]);
            for (int e = 0; e < A; e += 3) {
                Z.issue(pplanes, pscales, nb, loff, soff, s_jt[e + 2 < A ? e + 2 : last]);
                X.template consume<G, TOK>(s_jt[e], s_q[e], acc);
                X.issue(pplanes, pscales, nb, loff, soff, s_jt[e + 3 < A ? e + 3 : last]);
                if (e + 1 < A) Y.template consume<G, TOK>(s_jt[e + 1], s_q[e + 1], acc);
                Y.issue(pplanes, pscales, nb, loff, soff, s_jt[e + 4 < A ? e + 4 : last]);
                if (e + 2 < A) Z.template consume<G, TOK>(s_jt[e + 2], s_q[e + 2], acc);
            }
        } else {
            for (int e = 0; e < A; e += 2) {
                Y.issue(pplanes, pscales, nb, loff, soff, s_jt[e + 1 < A ? e + 1 : last]);
                X.template consume<G, TOK>(s_jt[e], s_q[e], acc);
                X.issue(pplanes, pscales, nb, loff, soff, s_jt[e + 2 < A ? e + 2 : last]);
                if (e + 1 < A) Y.template consume<G, TOK>(s_jt[e + 1], s_q[e + 1], acc);
            }
        }
    }

    const int64_t tok0 = blk * 64 + part * TOK;   // physical token of acc[0]
    if (MODE == kLaneMax) {
        // one value per lane and head: the max score of the lane's valid tokens
        if (lb >= a.nlb) return;
        const int64_t row = a.nlb * kParts;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < TOK; ++i)
                mx = (live && tok0 + i < a.n) ? fmaxf(mx, acc[h][i]) : mx;
            a.out[((size_t)p * G + h) * row + lb * kParts + part] = mx;
        }
    } else if (!FILTER) {
        const int64_t row = a.nlb * 64;
        const int64_t pos0 = lb * 64 + part * TOK;  // position in the output row
        if (lb >= a.nlb) return;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float* o = a.out + ((size_t)p * G + h) * row + pos0;
#pragma unroll
            for (int i = 0; i < TOK; i += 4) {
                float4 v;
                v.x = (live && tok0 + i + 0 < a.n) ? acc[h][i + 0] : -INFINITY;
                v.y = (live && tok0 + i + 1 < a.n) ? acc[h][i + 1] : -INFINITY;
                v.z = (live && tok0 + i + 2 < a.n) ? acc[h][i + 2] : -INFINITY;
                v.w = (live && tok0 + i + 3 < a.n) ? acc[h][i + 3] : -INFINITY;
                *reinterpret_cast<float4*>(o + i) = v;
            }
        }
    } else {
        // valid-token mask of the lane (only the last block is partial)
        const int64_t nvalid = a.n - tok0;
        const uint32_t vmask = !live || nvalid <= 0 ? 0u
                               : (nvalid >= TOK ? (TOK == 32 ? 0xFFFFFFFFu : 0xFFFFu)
                                                : ((1u << nvalid) - 1u));
        // survivors of every head: keep[h] bit i <=> token i's score >= threshold
        uint32_t keep[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const uint32_t tk = a.tau[(size_t)p * G + h];
            // threshold as a float; +0 becomes -0 so that s - th keeps -0 scores
            float th = tk <= 0x007FFFFFu ? -INFINITY : key_score(tk);
            if (th == 0.0f) th = -0.0f;
            // sign of fl(s - th) is 1 exactly when s < th: shift it into a mask
            uint32_t fail = 0;
#pragma unroll
            for (int i = TOK - 1; i >= 0; --i)
                fail = __builtin_amdgcn_alignbit(fail, __float_as_uint(acc[h][i] - th), 31);
            keep[h] = ~fail & vmask;
        }
        // slots: each lane's offset within the wavefront from one LDS
        // fetch-and-add per head, then one global fetch-and-add per head and
        // wavefront, all issued before any result is waited for
        uint32_t* wc = s_wcount[wave];
        if (lane < G) wc[lane] = 0u;
        uint32_t off[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const uint32_t cnt = __popc(keep[h]);
            off[h] = cnt ? atomicAdd(&wc[h], cnt) : 0u;
        }
        uint32_t base = 0;
        if (lane < G) {
            const uint32_t tot = wc[lane];
            if (tot) base = atomicAdd(&a.counts[(size_t)p * G + lane], tot);
        }
        float* stage = s_stage[wave][lane];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            uint32_t k = keep[h];
            const int64_t b0 = (int64_t)(uint32_t)__builtin_amdgcn_readlane((int)base, h) + off[h];
            if (k) {
#pragma unroll
                for (int i = 0; i < TOK; i += 4)
                    *reinterpret_cast<float4*>(stage + i) =
                        make_float4(acc[h][i], acc[h][i + 1], acc[h][i + 2], acc[h][i + 3]);
            }
            int64_t slot = b0;
            uint64_t* dst = a.cand + ((size_t)p * G + h) * a.cap;
            while (k) {
                const int i = __ffs(k) - 1;
                k &= k - 1;
                if (slot < a.cap) dst[slot] = composite(score_key(stage[i]), (uint32_t)(tok0 + i));
                ++slot;
            }
        }
    }
}

// blockIdx.y is the pair; with a pair list (score mode only), the rows of
// the grid take the listed pairs in turn instead.
template <int G, int TOK, int MODE>
__global__ __launch_bounds__(kScanThreads) void scan_kernel(ScanArgs a)
{
    if (MODE == kStore && a.list) {
        const uint32_t nlist = a.list[0];
        for (uint32_t r = blockIdx.y; r < nlist; r += gridDim.y) {
            scan_pair<G, TOK, MODE>(a, (int)a.list[1 + r]);
            __syncthreads();  // the pair's LDS tables are rewritten by the next one
        }
        return;
    }
    scan_pair<G, TOK, MODE>(a, (int)blockIdx.y);
}

template <int G, int MODE>
hipError_t launch_g(const ScanArgs& a, int P, hipStream_t st)
{
    constexpr int TOK = G <= 4 ? 32 : 16;
    constexpr int per_wg = (kScanThreads / kWave) * TOK;  // blocks per workgroup
    // a pair list is walked by kListRows rows of workgroups
    const int rows = a.list ? (P < kListRows ? P : kListRows) : P;
    dim3 grid((unsigned)((a.nlb + per_wg - 1) / per_wg), (unsigned)rows);
    scan_kernel<G, TOK, MODE><<<grid, kScanThreads, 0, st>>>(a);
    return hipGetLastError();
}

template <int MODE>
hipError_t launch_any(const ScanArgs& a, int P, int G, hipStream_t st)
{
    switch (G) {
    case 1: return launch_g<1, MODE>(a, P, st);
    case 2: return launch_g<2, MODE>(a, P, st);
    case 3: return launch_g<3, MODE>(a, P, st);
    case 4: return launch_g<4, MODE>(a, P, st);
    case 5: return launch_g<5, MODE>(a, P, st);
    case 6: return launch_g<6, MODE>(a, P, st);
    case 7: return launch_g<7, MODE>(a, P, st);
    default: return launch_g<8, MODE>(a, P, st);
    }
}

}  // namespace

hipError_t launch_scan_args(const ScanArgs& a, int P, int G, int mode, hipStream_t st)
{
    if (mode == kFilter) return launch_any<kFilter>(a, P, G, st);
    if (mode == kLaneMax) return launch_any<kLaneMax>(a, P, G, st);
    return launch_any<kStore>(a, P, G, st);
}

hipError_t launch_scan(const uint64_t* planes, const uint16_t* scales, int P, int D, int64_t n,
                       int64_t ldb, const uint8_t* depth, const int16_t* active,
                       const int32_t* n_active, const float* q_used, int G, float* scores,
                       hipStream_t st)
{
    ScanArgs a{};
    a.planes = planes;
    a.scales = scales;
    a.D = D;
    a.n = n;
    a.nb = (n + 63) / 64;
    a.ldb = ldb;
    a.depth = depth;
    a.active = active;
    a.n_active = n_active;
    a.q_used = q_used;
    a.stride = 1;
    a.nlb = a.nb;
    a.out = scores;
    return launch_any<kStore>(a, P, G, st);
}

}  // namespace fathom

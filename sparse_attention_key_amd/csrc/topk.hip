// Top-k per query head and union per KV head (yeyulingfeng.com write-up of
// Fathom: every query head keeps the k keys of highest approximate score;
// the group fetches the union of its G winner sets).
//
// Ordering: (score descending, token index ascending), -0 == +0.  Scores map
// to order-preserving 32-bit keys and then to 64-bit composites
// key << 32 | ~index, which are unique, so "the k largest composites" is the
// exact answer with ties already broken.
//
// Pipeline per call (one selection = one (pair, head)):
//  1. threshold: from a SAMPLE of scores (one run of 32 consecutive blocks
//     in every `stride` runs; in the fused path, the maxima of groups of 16
//     tokens of those blocks).  Each sample value is a distinct token's
//     score.  From materialised scores the k-th largest sample value is
//     used: a lower bound of the true k-th largest, so every true winner
//     passes it.  The fused path uses the ceil(2k / stride)-th largest, which
//     leaves about 2k candidates; should fewer than k pass, stage 3 selects
//     that head over all of its scores.  The bound used is the lower edge of
//     the 22-bit key bin holding the chosen sample value.
//  2. filter:    one pass over all scores appends key >= threshold to a
//                candidate list (workgroup-aggregated atomics; in the fused
//                path, inside the scan).
//  3. select:    exact k largest composites of the candidates (radix select
//                with 11-bit digits, the last levels in LDS), each winner
//                placed by its rank; a second rank by token index gives the
//                winners sorted by index.  A selection whose candidates
//                overflowed their capacity, or number fewer than k, runs the
//                same select directly over all its scores instead.
//  4. union:     merge of the G index-sorted lists of a pair, duplicates
//                dropped.
#include "common.h"

namespace fathom {
namespace {

constexpr int kSelThreads = 1024;
// Selections and the fused path's thresholds run 512 threads per
// workgroup: with a thousand or so candidates per selection (a few thousand
// sample values per threshold), more and smaller workgroups finish sooner
// (stage 3 at 1M tokens x 288 pairs: 0.100 -> 0.079 ms).  The kernels' code
// works for any multiple of 64 threads up to kSelThreads.
constexpr int kSelectThreads = 512;
constexpr int kBins = 2048;
constexpr int kBuf = 4096;

struct SelShared {
    uint32_t hist[2][kBins];  // level l counts into hist[l & 1] and clears the other
    uint64_t buf[kBuf + 8];   // + 8 zero pads after the winners for the linear rank loop
    uint64_t wlo[kSelThreads / kWave], whi[kSelThreads / kWave];
    uint32_t nbuf;
    uint32_t bin, above, inbin;
};

struct DenseSrc {
    const float* s;
    int64_t n;       // valid tokens
    int64_t stride;  // one run of 32 blocks in every `stride` runs (1 = all)
    int64_t count;   // elements enumerated
    __device__ __forceinline__ uint64_t get(int64_t e, bool& ok) const
    {
        const int64_t lb = e >> 6;
        const int64_t tok = ((lb >> 5) * stride * 32 + (lb & 31)) * 64 + (e & 63);
        ok = tok < n;
        const float v = ok ? s[tok] : 0.0f;
        return composite(score_key(v), (uint32_t)tok);
    }
};

struct CandSrc {
    const uint64_t* c;
    int64_t count;
    __device__ __forceinline__ uint64_t get(int64_t e, bool& ok) const
    {
        ok = true;
        return c[e];
    }
};

struct LdsSrc {
    const uint64_t* c;
    int64_t count;
    __device__ __forceinline__ uint64_t get(int64_t e, bool& ok) const
    {
        ok = true;
        return c[e];
    }
};

// Radix select over 64-bit values x below 2^bits, most significant digit
// first: 11-bit digits from bit `bits` down (the last one narrower).  The
// digits fixed so far form `prefix` under the contiguous top mask `pmask`;
// `need` is the rank (1 = largest) still sought among the values that match
// them.  Once the bin of the sought value holds it alone, the k largest are
// exactly the values whose masked x is at or above the prefix.  The values
// are the composites themselves (bits = 64), or their offsets from the
// smallest one (bits = the bit length of the range): then the first digit
// already spreads them over all bins, where the top bits of a selection's
// candidates are nearly all equal and their histogram would funnel every
// add into a few bins.
struct Radix {
    uint64_t prefix, pmask;
    int need, lvl, bits;
    __device__ __forceinline__ int hi() const { return bits - 11 * lvl; }  // digit covers [shift, hi)
    __device__ __forceinline__ int shift() const { return hi() > 11 ? hi() - 11 : 0; }
    __device__ __forceinline__ uint32_t mask() const { return (1u << (hi() - shift())) - 1u; }
    __device__ __forceinline__ bool done() const { return hi() <= 0; }
    __device__ __forceinline__ bool in(uint64_t x) const { return (x & pmask) == prefix; }
    __device__ __forceinline__ uint32_t digit(uint64_t x) const { return (uint32_t)(x >> shift()) & mask(); }
    __device__ __forceinline__ bool at_or_above(uint64_t x) const { return (x & pmask) >= prefix; }
};

// Zeroes the first level's histogram (followed by a barrier).
__device__ __forceinline__ Radix radix_start(int need, SelShared& sh)
{
    for (int i = threadIdx.x; i < kBins; i += blockDim.x) sh.hist[0][i] = 0;
    __syncthreads();
    return Radix{0, 0, need, 0, 64};
}

// Values every thread of the workgroup reads alike (from LDS), moved to
// scalar registers.
__device__ __forceinline__ uint32_t uniform_u32(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}

__device__ __forceinline__ uint64_t uniform_u64(uint64_t v)
{
    return ((uint64_t)uniform_u32((uint32_t)(v >> 32)) << 32) | uniform_u32((uint32_t)v);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m)
{
    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, m, kWave);
    const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), m, kWave);
    return ((uint64_t)hi << 32) | lo;
}

// Radix over offsets from the smallest element, `lo` (lo_t, hi_t: this
// thread's extremes; ~0 and 0 when it holds none).  Zeroes the first
// histogram.
__device__ Radix radix_start_range(int need, uint64_t lo_t, uint64_t hi_t, SelShared& sh,
                                   uint64_t& lo)
{
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
        const uint64_t a = shfl_xor_u64(lo_t, o), b = shfl_xor_u64(hi_t, o);
        lo_t = a < lo_t ? a : lo_t;
        hi_t = b > hi_t ? b : hi_t;
    }
    const int wave = threadIdx.x / kWave, nw = blockDim.x / kWave;
    if (lane_id() == 0) {
        sh.wlo[wave] = lo_t;
        sh.whi[wave] = hi_t;
    }
    for (int i = threadIdx.x; i < kBins; i += blockDim.x) sh.hist[0][i] = 0;
    __syncthreads();
    uint64_t hi = 0;
    lo = ~0ull;
    for (int w = 0; w < nw; ++w) {
        lo = sh.wlo[w] < lo ? sh.wlo[w] : lo;
        hi = sh.whi[w] > hi ? sh.whi[w] : hi;
    }
    lo = uniform_u64(lo);
    hi = uniform_u64(hi);
    const int bits = hi > lo ? 64 - __clzll((long long)(hi - lo)) : 1;
    return Radix{0, 0, need, 0, bits};
}

// Histogram of the current level; the next level's buffer is zeroed here
// (its last reader, the previous level's bin search, ended at a barrier).
__device__ __forceinline__ uint32_t* level_begin(const Radix& r, SelShared& sh)
{
    uint32_t* nxt = sh.hist[(r.lvl + 1) & 1];
    for (int i = threadIdx.x; i < kBins; i += blockDim.x) nxt[i] = 0;
    return sh.hist[r.lvl & 1];
}

// Inclusive prefix sum over the wavefront with DPP moves: shifts by 1, 2, 4
// and 8 within each row of 16 lanes (lanes shifted in from outside the row
// read 0), then row 0's total into row 1 and row 2's into row 3 (row_bcast
// 15), then rows 0-1's total into rows 2 and 3 (row_bcast 31).
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t x)
{
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true);  // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true);  // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true);  // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true);  // row_shr:8
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false); // row_bcast:15
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false); // row_bcast:31
    return x;
}

// After the histogram: the first wavefront finds the bin holding the
// need-th largest, then every thread fixes that digit.  Bins are taken top
// first: lane l sums bins 2047 - 32l down to 2016 - 32l, a wavefront prefix
// sum over those groups names the group that holds the sought element, and
// a second prefix sum over that group's 32 bins (one per lane) names the
// bin.  Returns the number of elements in the bin.
__device__ uint32_t level_end(Radix& r, SelShared& sh)
{
    __syncthreads();
    if (threadIdx.x < kWave) {
        const uint32_t* h = sh.hist[r.lvl & 1];
        const int lane = threadIdx.x;
        const uint4* h4 = reinterpret_cast<const uint4*>(h + kBins - 32 * (lane + 1));
        uint32_t sum = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint4 x = h4[j];
            sum += x.x + x.y + x.z + x.w;
        }
        const uint32_t need = (uint32_t)r.need;
        uint32_t inc = wave_incl_sum(sum);
        // the first group whose running total reaches need
        const int g = __builtin_ctzll(__ballot(inc >= need));
        const uint32_t before = (uint32_t)__shfl((int)(inc - sum), g, kWave);
        const int b = kBins - 1 - 32 * g - (lane & 31);  // lanes 32..63 repeat 0..31
        const uint32_t c = h[b];
        inc = before + wave_incl_sum(lane < 32 ? c : 0u);
        const int l = __builtin_ctzll(__ballot(lane < 32 && inc >= need));
        if (lane == l) {
            sh.bin = (uint32_t)b;
            sh.above = inc - c;
            sh.inbin = c;
        }
    }
    __syncthreads();
    const int sft = r.shift();
    r.need -= (int)uniform_u32(sh.above);
    r.prefix |= (uint64_t)uniform_u32(sh.bin) << sft;
    r.pmask |= (uint64_t)r.mask() << sft;
    ++r.lvl;
    return uniform_u32(sh.inbin);  // read before the next level's first barrier
}

// One radix level over src, four elements per thread loaded before any is
// counted.
template <class Src>
__device__ uint32_t radix_level(const Src& src, Radix& r, SelShared& sh)
{
    uint32_t* h = level_begin(r, sh);
    const int64_t bd = blockDim.x;
    for (int64_t e0 = threadIdx.x; e0 < src.count; e0 += 4 * bd) {
        uint64_t v[4];
        bool ok[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t e = e0 + u * bd;
            ok[u] = false;
            v[u] = e < src.count ? src.get(e, ok[u]) : 0;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (ok[u] && r.in(v[u])) atomicAdd(&h[r.digit(v[u])], 1u);
    }
    return level_end(r, sh);
}

// Radix levels over src until the sought element's bin fits in LDS; that
// bin is then copied to sh.buf and the remaining levels run there.
template <class Src>
__device__ Radix kth_largest(const Src& src, int need, SelShared& sh)
{
    Radix r = radix_start(need, sh);
    uint32_t inbin;
    do {
        inbin = radix_level(src, r, sh);
    } while (inbin > (uint32_t)kBuf && !r.done());
    if (inbin <= 1) return r;
    if (threadIdx.x == 0) sh.nbuf = 0;
    __syncthreads();
    for (int64_t e = threadIdx.x; e < src.count; e += blockDim.x) {
        bool ok;
        const uint64_t v = src.get(e, ok);
        if (ok && r.in(v)) {
            const uint32_t slot = atomicAdd(&sh.nbuf, 1u);
            if (slot < (uint32_t)kBuf) sh.buf[slot] = v;
        }
    }
    __syncthreads();
    const LdsSrc lsrc{sh.buf, (int64_t)inbin};
    while (!r.done() && inbin > 1) inbin = radix_level(lsrc, r, sh);
    return r;
}

// Up to kRegSlots candidates per thread held in registers: slot q of
// thread t is candidate q * blockDim + t.
constexpr int kRegSlots = 16;

struct RegCands {
    uint64_t v[kRegSlots];
    uint32_t valid;  // bit q: slot q holds a candidate
};

__device__ __forceinline__ void load_regs(const uint64_t* c, int64_t cnt, RegCands& rc)
{
    rc.valid = 0;
#pragma unroll
    for (int q = 0; q < kRegSlots; ++q) {
        const int64_t e = (int64_t)q * blockDim.x + threadIdx.x;
        const bool ok = e < cnt;
        rc.v[q] = ok ? c[e] : 0;
        rc.valid |= ok ? 1u << q : 0u;
    }
}

// Radix levels over the candidates in registers, which are replaced by
// their offsets from the smallest one (returned in `base`).
__device__ Radix kth_largest_regs(RegCands& rc, int need, SelShared& sh, uint64_t& base)
{
    uint64_t lo = ~0ull, hi = 0;
#pragma unroll
    for (int q = 0; q < kRegSlots; ++q)
        if ((rc.valid >> q) & 1u) {
            lo = rc.v[q] < lo ? rc.v[q] : lo;
            hi = rc.v[q] > hi ? rc.v[q] : hi;
        }
    Radix r = radix_start_range(need, lo, hi, sh, base);
#pragma unroll
    for (int q = 0; q < kRegSlots; ++q) {
        rc.v[q] -= base;
        // opaque to the optimiser: otherwise the winners' offset + base
        // folds back to the original value, which then stays live too
        asm volatile("" : "+v"(rc.v[q]));
    }
    for (;;) {
        uint32_t* h = level_begin(r, sh);
#pragma unroll
        for (int q = 0; q < kRegSlots; ++q)
            if (((rc.valid >> q) & 1u) && r.in(rc.v[q])) atomicAdd(&h[r.digit(rc.v[q])], 1u);
        if (level_end(r, sh) <= 1 || r.done()) break;
    }
    return r;
}

// Appends the candidates at or above the cut to sh.buf with one LDS atomic
// per wavefront: the wavefront's winners are counted first, then each is
// placed at the wavefront's base plus the winners before it (earlier slots,
// then lower lanes of its own slot).
__device__ __forceinline__ void winners_from_regs(const RegCands& rc, const Radix& r, uint64_t base,
                                                  SelShared& sh)
{
    const int lane = lane_id();
    uint32_t wins = 0, total = 0;
#pragma unroll
    for (int q = 0; q < kRegSlots; ++q) {
        const bool win = ((rc.valid >> q) & 1u) && r.at_or_above(rc.v[q]);
        wins |= win ? 1u << q : 0u;
        total += (uint32_t)__popcll(__ballot(win));
    }
    uint32_t slot = 0;
    if (lane == 0 && total != 0) slot = atomicAdd(&sh.nbuf, total);
    slot = (uint32_t)__shfl((int)slot, 0, kWave);
#pragma unroll
    for (int q = 0; q < kRegSlots; ++q) {
        const bool win = (wins >> q) & 1u;
        const uint64_t b = __ballot(win);
        if (win) sh.buf[slot + (uint32_t)__popcll(b & lanes_below(lane))] = rc.v[q] + base;
        slot += (uint32_t)__popcll(b);
    }
}

__device__ __forceinline__ uint32_t shfl_xor_any(uint32_t v, int m)
{
    return (uint32_t)__shfl_xor((int)v, m, kWave);
}

__device__ __forceinline__ uint64_t shfl_xor_any(uint64_t v, int m)
{
    const uint32_t lo = shfl_xor_any((uint32_t)v, m), hi = shfl_xor_any((uint32_t)(v >> 32), m);
    return ((uint64_t)hi << 32) | lo;
}

// Bitonic sort of one value per lane across the wavefront, descending by
// lane: in every merge step the lane of each exchanged pair that lies in a
// descending run of the current size keeps the larger value at the lower
// lane (the last run spans the wavefront, so the result is descending).
template <class T>
__device__ __forceinline__ T wave_sort_desc(T v)
{
    const int lane = lane_id();
#pragma unroll
    for (int size = 2; size <= kWave; size <<= 1) {
#pragma unroll
        for (int st = size >> 1; st > 0; st >>= 1) {
            const T o = shfl_xor_any(v, st);
            const bool keep_max = ((lane & size) == 0) == ((lane & st) == 0);
            const T hi = v > o ? v : o, lo = v > o ? o : v;
            v = keep_max ? hi : lo;
        }
    }
    return v;
}

// Number of entries above x in nch chunks of 64, each sorted descending:
// per chunk, binary lifting over the first 63 positions then one read of the
// position reached (which exceeds x only when all 64 do).  Eight chunks'
// searches run interleaved.
template <class T>
__device__ __forceinline__ int count_above(const T* a, int nch, T x)
{
    int r = 0;
    for (int c0 = 0; c0 < nch; c0 += 8) {
        int base[8], pos[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            base[q] = (c0 + q < nch ? c0 + q : nch - 1) * kWave;
            pos[q] = 0;
        }
#pragma unroll
        for (int st = kWave / 2; st > 0; st >>= 1)
#pragma unroll
            for (int q = 0; q < 8; ++q) pos[q] += a[base[q] + pos[q] + st - 1] > x ? st : 0;
#pragma unroll
        for (int q = 0; q < 8; ++q)
            if (c0 + q < nch) r += pos[q] + (a[base[q] + pos[q]] > x ? 1 : 0);
    }
    return r;
}

// The pairs with some head whose candidates overflowed their capacity, in
// pair order: list[0] = how many, list[1..] = the pairs.  One workgroup.
__global__ __launch_bounds__(kSelThreads) void overflow_list_kernel(const uint32_t* __restrict__ counts,
                                                                   int P, int G, int64_t cap, int k,
                                                                   uint32_t* __restrict__ list)
{
    __shared__ uint32_t wsum[kSelThreads / kWave];
    const int lane = lane_id(), wave = threadIdx.x / kWave, nw = blockDim.x / kWave;
    uint32_t base = 0;
    for (int p0 = 0; p0 < P; p0 += blockDim.x) {
        const int p = p0 + (int)threadIdx.x;
        bool f = false;
        if (p < P)
            for (int h = 0; h < G; ++h) {
                const int64_t c = counts[(size_t)p * G + h];
                f |= c > cap || c < (int64_t)k;
            }
        const uint64_t b = __ballot(f);
        if (lane == 0) wsum[wave] = (uint32_t)__popcll(b);
        __syncthreads();
        uint32_t off = base, all = 0;
        for (int w = 0; w < nw; ++w) {
            off += w < wave ? wsum[w] : 0u;
            all += wsum[w];
        }
        if (f) list[1 + off + (uint32_t)__popcll(b & lanes_below(lane))] = (uint32_t)p;
        base += all;
        __syncthreads();  // wsum is rewritten by the next round
    }
    if (threadIdx.x == 0) list[0] = base;
}

__global__ __launch_bounds__(kSelThreads) void threshold_kernel(const float* __restrict__ scores,
                                                                int64_t n, int64_t npad,
                                                                int64_t stride, int64_t count,
                                                                int64_t valid, int k,
                                                                uint32_t* __restrict__ tau,
                                                                uint32_t* __restrict__ counts)
{
    __shared__ SelShared sh;
    const int64_t m = blockIdx.x;
    if (threadIdx.x == 0) counts[m] = 0u;  // the selection's candidate count, for the filter that follows
    if (valid < k) {
        if (threadIdx.x == 0) tau[m] = 0u;
        return;
    }
    // Any lower bound of the k-th largest score is a valid threshold: two
    // 11-bit radix levels locate the bin (the top 22 bits of the key) that
    // holds the sample's k-th largest, and its lower edge is used -- within
    // 2^-14 of that value, and every element of the bin is at or above it.
    DenseSrc src{scores + m * npad, n, stride, count};
    Radix r = radix_start(k, sh);
    radix_level(src, r, sh);
    radix_level(src, r, sh);
    if (threadIdx.x == 0) tau[m] = (uint32_t)(r.prefix >> 32);
}

// Candidates of one (selection, 4096-token chunk).  blockIdx.x is the
// selection, so neighbouring workgroups feed different counters; each
// workgroup stages its survivors in LDS and takes its slots with a single
// global atomic.
__global__ __launch_bounds__(256) void filter_kernel(const float* __restrict__ scores, int64_t n,
                                                     int64_t npad, const uint32_t* __restrict__ tau,
                                                     uint32_t* __restrict__ counts,
                                                     uint64_t* __restrict__ cand, int64_t cap)
{
    constexpr int kItems = 16;
    __shared__ uint64_t s_c[256 * kItems];
    __shared__ uint32_t s_n, s_base;
    const int64_t m = blockIdx.x;
    const uint32_t th = tau[m];
    const float* s = scores + m * npad;
    const int64_t chunks = (npad + 256 * kItems - 1) / (256 * kItems);
    for (int64_t c = blockIdx.y; c < chunks; c += gridDim.y) {
        const int64_t base = c * (256 * kItems);
        if (threadIdx.x == 0) s_n = 0;
        __syncthreads();
        float v[kItems];
#pragma unroll
        for (int r = 0; r < kItems; ++r) {  // all loads in flight before any test
            const int64_t tok = base + r * 256 + threadIdx.x;
            v[r] = tok < n ? s[tok] : -INFINITY;
        }
#pragma unroll
        for (int r = 0; r < kItems; ++r) {
            const int64_t tok = base + r * 256 + threadIdx.x;
            const uint32_t key = score_key(v[r]);
            if (tok < n && key >= th) s_c[atomicAdd(&s_n, 1u)] = composite(key, (uint32_t)tok);
        }
        __syncthreads();
        const uint32_t cnt = s_n;  // uniform over the workgroup
        if (cnt != 0) {
            if (threadIdx.x == 0) s_base = atomicAdd(&counts[m], cnt);
            __syncthreads();
            const int64_t b0 = s_base;
            for (uint32_t i = threadIdx.x; i < cnt; i += 256)
                if (b0 + i < cap) cand[m * cap + b0 + i] = s_c[i];
        }
        __syncthreads();  // s_c, s_n and s_base are reused by the next chunk
    }
}

// Eight waves per SIMD: two workgroups per CU.
__global__ __launch_bounds__(kSelectThreads, 6) void select_kernel(
    const float* __restrict__ scores, int64_t n, int64_t npad, const uint32_t* __restrict__ counts,
    const uint64_t* __restrict__ cand, int64_t cap, int k, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_val, int32_t* __restrict__ sorted_idx)
{
    __shared__ SelShared sh;
    const int64_t m = blockIdx.x;
    const int64_t cnt = counts[m];
    // too many candidates for the buffer, or (fused path) fewer than k
    // above a statistical threshold: select over all scores instead
    const bool dense = cnt > cap || cnt < (int64_t)k;
    if (!dense && cnt <= (int64_t)kRegSlots * blockDim.x) {
        // candidates read once into registers; the radix levels and the
        // winner gather run from there
        RegCands rc;
        uint64_t base;
        load_regs(cand + m * cap, cnt, rc);
        const Radix r = kth_largest_regs(rc, k, sh, base);
        if (threadIdx.x == 0) sh.nbuf = 0;
        __syncthreads();
        winners_from_regs(rc, r, base, sh);
    } else {
        DenseSrc dsrc{scores + m * npad, n, 1, npad};
        CandSrc csrc{cand + m * cap, cnt};
        const Radix r = dense ? kth_largest(dsrc, k, sh) : kth_largest(csrc, k, sh);
        if (threadIdx.x == 0) sh.nbuf = 0;
        __syncthreads();
        const int64_t total = dense ? dsrc.count : csrc.count;
        for (int64_t e = threadIdx.x; e < total; e += blockDim.x) {
            bool ok;
            const uint64_t v = dense ? dsrc.get(e, ok) : csrc.get(e, ok);
            if (ok && r.at_or_above(v)) {
                const uint32_t slot = atomicAdd(&sh.nbuf, 1u);
                if (slot < (uint32_t)kBuf) sh.buf[slot] = v;
            }
        }
    }
    __syncthreads();
    // Place each winner by its rank among the k by composite (its output
    // position) and by token index (its position in the index-sorted list
    // the union merges); index i < index j exactly when ~i > ~j in the low
    // word.
    if (k <= kBins) {
        // Merge ranking: every wave sorts 64-winner chunks descending in
        // registers (composites in place in buf, low words into hist, which
        // the radix levels no longer need); a winner's rank is then the sum
        // over all chunks of how many entries exceed it, a 7-read binary
        // search per chunk.  Zero pads fill the last chunk: a composite's
        // low word is ~index with index < 2^31, so every real composite and
        // every real low word is nonzero and the pads count below them all.
        const int nch = (k + kWave - 1) / kWave;
        for (int i = k + (int)threadIdx.x; i < nch * kWave; i += blockDim.x) sh.buf[i] = 0;
        __syncthreads();
        const int lane = lane_id();
        for (int c = (int)(threadIdx.x / kWave); c < nch; c += (int)(blockDim.x / kWave)) {
            const uint64_t v = sh.buf[c * kWave + lane];
            const uint64_t sv = wave_sort_desc(v);
            const uint32_t sl = wave_sort_desc((uint32_t)v);
            sh.buf[c * kWave + lane] = sv;
            sh.hist[0][c * kWave + lane] = sl;
        }
        __syncthreads();
        for (int t = threadIdx.x; t < 2 * nch * kWave; t += blockDim.x) {
            const bool by_index = t >= nch * kWave;
            const int slot = by_index ? t - nch * kWave : t;
            // sorted slot (chunk c, position p) holds a winner iff p < k - c * 64
            if (slot >= k) continue;
            if (!by_index) {
                const uint64_t v = sh.buf[slot];
                const int r = count_above(sh.buf, nch, v);
                topk_idx[m * k + r] = (int32_t)(~(uint32_t)v);
                if (topk_val) topk_val[m * k + r] = key_score((uint32_t)(v >> 32));
            } else {
                const uint32_t lo = sh.hist[0][slot];
                sorted_idx[m * k + count_above(sh.hist[0], nch, lo)] = (int32_t)(~lo);
            }
        }
    } else {
        // Linear ranking, eight LDS reads in flight per step; eight zero pads
        // after the k winners rank below every composite and every index.
        if (threadIdx.x < 8) sh.buf[k + threadIdx.x] = 0;
        __syncthreads();
        for (int i = threadIdx.x; i < k; i += blockDim.x) {
            const uint64_t v = sh.buf[i];
            const uint32_t lo = (uint32_t)v;
            int r = 0, ri = 0;
            for (int j = 0; j < k; j += 8) {
                uint64_t u[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) u[q] = sh.buf[j + q];
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    r += u[q] > v ? 1 : 0;
                    ri += (uint32_t)u[q] > lo ? 1 : 0;
                }
            }
            topk_idx[m * k + r] = (int32_t)(~lo);
            if (topk_val) topk_val[m * k + r] = key_score((uint32_t)(v >> 32));
            sorted_idx[m * k + ri] = (int32_t)(~lo);
        }
    }
}

// Union of the G winner lists of a pair, each sorted by token index: every
// element's place in the merged order is its own position plus the number
// of elements of each other list that precede it (binary search; equal
// indices ordered by list), then adjacent duplicates are dropped.
template <int G>
__global__ __launch_bounds__(kSelThreads) void union_kernel(const int32_t* __restrict__ sorted_idx,
                                                            int k,
                                                            int32_t* __restrict__ union_idx,
                                                            int32_t* __restrict__ union_len)
{
    constexpr int kPer = kMaxUnion / kSelThreads;
    __shared__ int32_t a[kMaxUnion];
    __shared__ uint32_t wsum[kSelThreads / kWave];
    const int p = blockIdx.x;
    const int total = G * k;
    const int32_t* src = sorted_idx + (size_t)p * total;
    for (int i = threadIdx.x; i < total; i += blockDim.x) a[i] = src[i];
    __syncthreads();
    int32_t val[kPer];
    int pos[kPer];
    // binary lifting over each other list, steps from the largest power of
    // two not above k; the G - 1 searches of an element run interleaved
    const int top = 1 << (31 - __clz(k));
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        pos[u] = -1;
        val[u] = 0;
        if (u * (int)blockDim.x >= total) continue;
        const int e = threadIdx.x + u * (int)blockDim.x;
        if (e < total) {
            const int h = e / k;
            const int32_t x = a[e];
            int cnt[G];
#pragma unroll
            for (int h2 = 0; h2 < G; ++h2) cnt[h2] = 0;
            for (int st = top; st > 0; st >>= 1) {
#pragma unroll
                for (int h2 = 0; h2 < G; ++h2) {
                    const int np = cnt[h2] + st;
                    if (h2 != h && np <= k) {
                        const int32_t y = a[h2 * k + np - 1];
                        if (h2 < h ? y <= x : y < x) cnt[h2] = np;
                    }
                }
            }
            int r = e - h * k;
#pragma unroll
            for (int h2 = 0; h2 < G; ++h2) r += h2 != h ? cnt[h2] : 0;
            val[u] = x;
            pos[u] = r;
        }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kPer; ++u)
        if (pos[u] >= 0) a[pos[u]] = val[u];
    __syncthreads();
    // each thread owns a contiguous run of the merged order; first
    // occurrences are counted, scanned and written out
    const int per = (total + blockDim.x - 1) / blockDim.x;
    const int beg = threadIdx.x * per;
    uint32_t cnt = 0;
    for (int i = beg; i < beg + per && i < total; ++i)
        cnt += (i == 0 || a[i] != a[i - 1]) ? 1u : 0u;
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    const uint32_t x = wave_incl_sum(cnt);
    if (lane == kWave - 1) wsum[wave] = x;
    __syncthreads();
    uint32_t off = 0, all = 0;
    for (int w = 0; w < (int)(blockDim.x / kWave); ++w) {
        if (w < wave) off += wsum[w];
        all += wsum[w];
    }
    uint32_t q = off + x - cnt;
    int32_t* out = union_idx + (size_t)p * total;
    for (int i = beg; i < beg + per && i < total; ++i)
        if (i == 0 || a[i] != a[i - 1]) out[q++] = a[i];
    for (int i = (int)all + threadIdx.x; i < total; i += blockDim.x) out[i] = -1;
    if (threadIdx.x == 0) union_len[p] = (int32_t)all;
}

// the union for G lists of k (the list count fixed at compile time, so the
// searches over the other lists unroll without per-list tests)
void launch_union(const int32_t* sorted, int P, int G, int k, int32_t* union_idx, int32_t* union_len,
                  hipStream_t st)
{
    const dim3 grid((unsigned)P);
    switch (G) {
    case 1: union_kernel<1><<<grid, kSelThreads, 0, st>>>(sorted, k, union_idx, union_len); break;
    case 2: union_kernel<2><<<grid, kSelThreads, 0, st>>>(sorted, k, union_idx, union_len); break;
    case 3: union_kernel<3><<<grid, kSelThreads, 0, st>>>(sorted, k, union_idx, union_len); break;
    case 4: union_kernel<4><<<grid, kSelThreads, 0, st>>>(sorted, k, union_idx, union_len); break;
    case 5: union_kernel<5><<<grid, kSelThreads, 0, st>>>(sorted, k, union_idx, union_len); break;
    case 6: union_kernel<6><<<grid, kSelThreads, 0, st>>>(sorted, k, union_idx, union_len); break;
    case 7: union_kernel<7><<<grid, kSelThreads, 0, st>>>(sorted, k, union_idx, union_len); break;
    default: union_kernel<8><<<grid, kSelThreads, 0, st>>>(sorted, k, union_idx, union_len); break;
    }
}

}  // namespace

TopkLayout topk_layout(int P, int G, int64_t n, int k)
{
    TopkLayout L{};
    const int64_t nb = (n + 63) / 64;
    L.m = (int64_t)P * G;
    // sample stride: ~sqrt(n / 4k) blocks (power of two), so the sample and
    // the expected candidate count (~k * stride) stay balanced
    int64_t s = 1;
    while ((s * 2) * (s * 2) * 4 * (int64_t)k <= n && s * 2 <= nb) s *= 2;
    L.stride = s;
    // maxima of groups of 16 tokens (four per block) carry almost the same
    // tail information as the tokens themselves once there are >= 8k of them
    L.lanemax = n >= 128 * (int64_t)k * s;
    // the fused threshold is the rank-th largest sample value: with one run
    // in every s sampled, about rank * s >= 2k scores lie above it.  That is
    // a statistical bound; a selection that ends up with fewer than k
    // candidates is selected over all of its scores instead (stage 3).
    L.rank = s == 1 ? k : (int)((2 * (int64_t)k + s - 1) / s);
    L.cap = 8 * (int64_t)k * s + 1024;
    if (L.cap > nb * 64) L.cap = nb * 64;
    L.sample_nlb = ((nb + 32 * s - 1) / (32 * s)) * 32;
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    L.off_tau = 0;
    L.off_count = up((size_t)L.m * 4);
    L.off_cand = up(L.off_count + (size_t)L.m * 4);
    L.off_sorted = up(L.off_cand + (size_t)L.m * (size_t)L.cap * 8);
    L.bytes = L.off_sorted + (size_t)L.m * (size_t)k * 4;
    L.off_list = up(L.bytes);
    L.off_sample = up(L.off_list + ((size_t)P + 1) * 4);
    L.off_repair = up(L.off_sample + (size_t)L.m * (size_t)L.sample_nlb * 64 * 4);
    L.bytes_fused = L.off_repair + (size_t)L.m * (size_t)nb * 64 * 4;
    return L;
}

hipError_t launch_topk(const float* scores, int P, int G, int64_t n, int k, int32_t* topk_idx,
                       float* topk_val, int32_t* union_idx, int32_t* union_len, void* ws,
                       const TopkLayout& L, hipStream_t st)
{
    const int64_t nb = (n + 63) / 64, npad = nb * 64;
    char* w = (char*)ws;
    uint32_t* tau = (uint32_t*)(w + L.off_tau);
    uint32_t* counts = (uint32_t*)(w + L.off_count);
    uint64_t* cand = (uint64_t*)(w + L.off_cand);
    int64_t valid = 0;  // sampled tokens below n
    for (int64_t b0 = 0; b0 < nb; b0 += 32 * L.stride) {
        const int64_t lo = b0 * 64, hi = (b0 + 32) * 64 < n ? (b0 + 32) * 64 : n;
        valid += hi - lo;
    }

    // (a sample of whole blocks' scores, 16x the fused path's: 1024 threads)
    threshold_kernel<<<dim3((unsigned)L.m), kSelThreads, 0, st>>>(scores, n, npad, L.stride,
                                                              L.sample_nlb * 64, valid, k, tau, counts);
    {
        // chunks of 4096 scores on grid.y, looped inside once there are more
        // than enough workgroups to fill the chip (grid.y stays below 65536)
        const int64_t chunks = (npad + 4095) / 4096;
        int64_t gy = (16384 + L.m - 1) / L.m;
        gy = gy < 64 ? 64 : gy > 65535 ? 65535 : gy;
        gy = gy < chunks ? gy : chunks;
        filter_kernel<<<dim3((unsigned)L.m, (unsigned)gy), 256, 0, st>>>(scores, n, npad, tau,
                                                                           counts, cand, L.cap);
    }
    int32_t* sorted = (int32_t*)(w + L.off_sorted);
    select_kernel<<<dim3((unsigned)L.m), kSelectThreads, 0, st>>>(scores, n, npad, counts, cand, L.cap,
                                                              k, topk_idx, topk_val, sorted);
    launch_union(sorted, P, G, k, union_idx, union_len, st);
    return hipGetLastError();
}

hipError_t launch_scan_topk(const ScanArgs& base, int P, int G, int k, int32_t* topk_idx,
                            float* topk_val, int32_t* union_idx, int32_t* union_len, void* ws,
                            const TopkLayout& L, int stages, hipStream_t st)
{
    const int64_t n = base.n, nb = base.nb, npad = nb * 64;
    char* w = (char*)ws;
    uint32_t* tau = (uint32_t*)(w + L.off_tau);
    uint32_t* counts = (uint32_t*)(w + L.off_count);
    uint64_t* cand = (uint64_t*)(w + L.off_cand);
    uint32_t* list = (uint32_t*)(w + L.off_list);
    float* sample = (float*)(w + L.off_sample);
    float* repair = (float*)(w + L.off_repair);
    hipError_t e;
    ScanArgs a = base;

    if (stages & 1) {
        // threshold: scores of every stride-th block, exact k-th largest (the
        // threshold kernel also clears the candidate counts)
        a.stride = L.stride;
        a.nlb = L.sample_nlb;
        a.out = sample;
        a.list = nullptr;
        if ((e = launch_scan_args(a, P, G, L.lanemax ? 2 : 0, st)) != hipSuccess) return e;
        // every lane maximum is a distinct token's score, so the k-th largest
        // of them is still a lower bound of the k-th largest score
        const int64_t row = L.sample_nlb * (L.lanemax ? 4 : 64);
        threshold_kernel<<<dim3((unsigned)L.m), kSelectThreads, 0, st>>>(sample, row, row, 1, row, row,
                                                                     L.rank, tau, counts);
    }
    if (stages & 2) {
        // filter: every block, keeping the scores at or above the threshold
        a = base;
        a.stride = 1;
        a.nlb = nb;
        a.tau = tau;
        a.counts = counts;
        a.cand = cand;
        a.cap = L.cap;
        a.list = nullptr;
        if ((e = launch_scan_args(a, P, G, 1, st)) != hipSuccess) return e;
    }
    if (stages & 4) {
        // pairs whose candidates overflowed get their full scores recomputed
        overflow_list_kernel<<<dim3(1), kSelThreads, 0, st>>>(counts, P, G, L.cap, k, list);
        a = base;
        a.stride = 1;
        a.nlb = nb;
        a.out = repair;
        a.list = list;
        if ((e = launch_scan_args(a, P, G, 0, st)) != hipSuccess) return e;
        // exact top-k of the candidates (or of the repaired scores), union
        int32_t* sorted = (int32_t*)(w + L.off_sorted);
        select_kernel<<<dim3((unsigned)L.m), kSelectThreads, 0, st>>>(repair, n, npad, counts, cand,
                                                                  L.cap, k, topk_idx, topk_val, sorted);
        launch_union(sorted, P, G, k, union_idx, union_len, st);
    }
    return hipGetLastError();
}

}  // namespace fathom

// Exact radix selection over 64-bit composites (score key << 32 | ~token),
// shared by the top-k kernels and the scan's repair kernel.  Device code
// only; every definition is internal to the including translation unit.
#pragma once

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

// KB: capacity of buf, which holds the winners (k <= KB) and the bin a
// radix level narrows a long source down to.  The full size serves every k
// up to 4096; the small one (k <= 2048) takes 33 KB instead of 49 KB, so
// four selection workgroups fit on a CU instead of three.
template <int KB>
struct SelSharedT {
    static constexpr int kCap = KB;
    uint32_t hist[2][kBins];  // level l counts into hist[l & 1] and clears the other
    uint64_t buf[KB + 8];     // + 8 zero pads after the winners for the linear rank loop
    uint64_t wlo[kSelThreads / kWave], whi[kSelThreads / kWave];
    uint32_t nbuf;
    uint32_t bin, above, inbin;
};
using SelShared = SelSharedT<4096>;
using SelSharedSmall = SelSharedT<2048>;
// the threshold kernels count radix levels only and never fill buf
using SelSharedHist = SelSharedT<8>;

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
template <class SH>
__device__ __forceinline__ Radix radix_start(int need, SH& sh)
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
template <class SH>
__device__ Radix radix_start_range(int need, uint64_t lo_t, uint64_t hi_t, SH& sh,
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
template <class SH>
__device__ __forceinline__ uint32_t* level_begin(const Radix& r, SH& sh)
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
template <class SH>
__device__ uint32_t level_end(Radix& r, SH& sh)
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
template <class Src, class SH>
__device__ uint32_t radix_level(const Src& src, Radix& r, SH& sh)
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
template <class Src, class SH>
__device__ Radix kth_largest(const Src& src, int need, SH& sh)
{
    Radix r = radix_start(need, sh);
    uint32_t inbin;
    do {
        inbin = radix_level(src, r, sh);
    } while (inbin > (uint32_t)SH::kCap && !r.done());
    if (inbin <= 1) return r;
    if (threadIdx.x == 0) sh.nbuf = 0;
    __syncthreads();
    for (int64_t e = threadIdx.x; e < src.count; e += blockDim.x) {
        bool ok;
        const uint64_t v = src.get(e, ok);
        if (ok && r.in(v)) {
            const uint32_t slot = atomicAdd(&sh.nbuf, 1u);
            if (slot < (uint32_t)SH::kCap) sh.buf[slot] = v;
        }
    }
    __syncthreads();
    const LdsSrc lsrc{sh.buf, (int64_t)inbin};
    while (!r.done() && inbin > 1) inbin = radix_level(lsrc, r, sh);
    return r;
}

// Up to NS candidates per thread held in registers: slot q of thread t is
// candidate q * blockDim + t.
template <int NS>
struct RegCands {
    uint64_t v[NS];
    uint32_t valid;  // bit q: slot q holds a candidate
};

template <int NS>
__device__ __forceinline__ void load_regs(const uint64_t* c, int64_t cnt, RegCands<NS>& rc)
{
    rc.valid = 0;
#pragma unroll
    for (int q = 0; q < NS; ++q) {
        const int64_t e = (int64_t)q * blockDim.x + threadIdx.x;
        const bool ok = e < cnt;
        rc.v[q] = ok ? c[e] : 0;
        rc.valid |= ok ? 1u << q : 0u;
    }
}

// Radix levels over the candidates in registers, which are replaced by
// their offsets from the smallest one (returned in `base`).
template <int NS, class SH>
__device__ Radix kth_largest_regs(RegCands<NS>& rc, int need, SH& sh, uint64_t& base)
{
    uint64_t lo = ~0ull, hi = 0;
#pragma unroll
    for (int q = 0; q < NS; ++q)
        if ((rc.valid >> q) & 1u) {
            lo = rc.v[q] < lo ? rc.v[q] : lo;
            hi = rc.v[q] > hi ? rc.v[q] : hi;
        }
    Radix r = radix_start_range(need, lo, hi, sh, base);
#pragma unroll
    for (int q = 0; q < NS; ++q) {
        rc.v[q] -= base;
        // opaque to the optimiser: otherwise the winners' offset + base
        // folds back to the original value, which then stays live too
        asm volatile("" : "+v"(rc.v[q]));
    }
    for (;;) {
        uint32_t* h = level_begin(r, sh);
#pragma unroll
        for (int q = 0; q < NS; ++q)
            if (((rc.valid >> q) & 1u) && r.in(rc.v[q])) atomicAdd(&h[r.digit(rc.v[q])], 1u);
        if (level_end(r, sh) <= 1 || r.done()) break;
    }
    return r;
}

// Appends the candidates at or above the cut to sh.buf with one LDS atomic
// per wavefront: the wavefront's winners are counted first, then each is
// placed at the wavefront's base plus the winners before it (earlier slots,
// then lower lanes of its own slot).
template <int NS, class SH>
__device__ __forceinline__ void winners_from_regs(const RegCands<NS>& rc, const Radix& r, uint64_t base,
                                                  SH& sh)
{
    const int lane = lane_id();
    uint32_t wins = 0, total = 0;
#pragma unroll
    for (int q = 0; q < NS; ++q) {
        const bool win = ((rc.valid >> q) & 1u) && r.at_or_above(rc.v[q]);
        wins |= win ? 1u << q : 0u;
        total += (uint32_t)__popcll(__ballot(win));
    }
    uint32_t slot = 0;
    if (lane == 0 && total != 0) slot = atomicAdd(&sh.nbuf, total);
    slot = (uint32_t)__shfl((int)slot, 0, kWave);
#pragma unroll
    for (int q = 0; q < NS; ++q) {
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

// Exact top-k of one selection m, written to topk_idx / topk_val (by rank)
// and sorted_idx (by token index): from its cnt candidates (cand, at most
// cap), or, when `dense`, from its full score row (n tokens of npad).
// NS: register slots per thread for the candidates; k <= SH::kCap.
template <int NS = 16, class SH>
__device__ void select_one(const float* __restrict__ srow, int64_t n, int64_t npad, bool dense,
                           const uint64_t* __restrict__ crow, int64_t cnt, int k, int64_t m,
                           int32_t* __restrict__ topk_idx, float* __restrict__ topk_val,
                           int32_t* __restrict__ sorted_idx, SH& sh)
{
    if (!dense && cnt <= (int64_t)NS * blockDim.x) {
        // candidates read once into registers; the radix levels and the
        // winner gather run from there
        RegCands<NS> rc;
        uint64_t base;
        load_regs(crow, cnt, rc);
        const Radix r = kth_largest_regs(rc, k, sh, base);
        if (threadIdx.x == 0) sh.nbuf = 0;
        __syncthreads();
        winners_from_regs(rc, r, base, sh);
    } else {
        DenseSrc dsrc{srow, n, 1, npad};
        CandSrc csrc{crow, cnt};
        const Radix r = dense ? kth_largest(dsrc, k, sh) : kth_largest(csrc, k, sh);
        if (threadIdx.x == 0) sh.nbuf = 0;
        __syncthreads();
        const int64_t total = dense ? dsrc.count : csrc.count;
        for (int64_t e = threadIdx.x; e < total; e += blockDim.x) {
            bool ok;
            const uint64_t v = dense ? dsrc.get(e, ok) : csrc.get(e, ok);
            if (ok && r.at_or_above(v)) {
                const uint32_t slot = atomicAdd(&sh.nbuf, 1u);
                if (slot < (uint32_t)SH::kCap) sh.buf[slot] = v;
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

}  // namespace
}  // namespace fathom

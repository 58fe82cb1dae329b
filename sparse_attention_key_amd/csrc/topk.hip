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
//  1. threshold: a lower bound of the k-th largest of a SAMPLE of scores
//     (one run of 32 consecutive blocks in every `stride` runs; in the fused
//     path, the maximum of each lane's 32 or 16 tokens of those blocks).
//     Each sample value is a distinct token's score, so the k-th largest
//     sample value -- and anything below it -- is a lower bound of the true
//     k-th largest: every true winner passes it.  The bound used is the
//     lower edge of the 22-bit key bin holding the sample's k-th largest.
//  2. filter:    one pass over all scores appends key >= threshold to a
//                candidate list (wavefront-aggregated atomics).
//  3. select:    exact k largest composites of the candidates (radix select
//                with 11-bit digits, the last levels in LDS), each winner
//                placed by its rank; a second rank by token index gives the
//                winners sorted by index.  A selection whose candidates
//                overflowed their capacity runs the same select directly over
//                all its scores instead.
//  4. union:     merge of the G index-sorted lists of a pair, duplicates
//                dropped.
#include "common.h"

namespace fathom {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kBins = 2048;
constexpr int kBuf = 4096;

struct SelShared {
    uint32_t hist[kBins];
    uint64_t buf[kBuf + 8];  // + 8 zero pads after the winners for the linear rank loop
    uint32_t wsum[kSelThreads / kWave];
    uint32_t nbuf;
    uint32_t bin, above, inbin;
    uint64_t result;
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

// Exclusive scan of one value per thread across the workgroup.
__device__ uint32_t block_excl_scan(uint32_t v, SelShared& sh)
{
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    uint32_t x = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const uint32_t y = __shfl_up(x, o, kWave);
        if (lane >= o) x += y;
    }
    if (lane == kWave - 1) sh.wsum[wave] = x;
    __syncthreads();
    uint32_t off = 0;
    for (int w = 0; w < wave; ++w) off += sh.wsum[w];
    __syncthreads();
    return off + x - v;
}

// One radix level: histogram of the 11-bit digit at `sft` over the elements
// matching (prefix, pmask); picks the bin holding the need-th largest and
// narrows prefix/pmask/need.  Returns the number of elements in that bin.
template <class Src>
__device__ uint32_t radix_level(const Src& src, int sft, uint32_t wm, uint64_t& prefix,
                                uint64_t& pmask, int& need, SelShared& sh)
{
    for (int i = threadIdx.x; i < kBins; i += blockDim.x) sh.hist[i] = 0;
    if (threadIdx.x == 0) {
        sh.bin = 0;
        sh.above = 0;
        sh.inbin = 0;
    }
    __syncthreads();
    for (int64_t e = threadIdx.x; e < src.count; e += blockDim.x) {
        bool ok;
        const uint64_t v = src.get(e, ok);
        if (ok && (v & pmask) == prefix) atomicAdd(&sh.hist[(uint32_t)(v >> sft) & wm], 1u);
    }
    __syncthreads();
    // reversed bins 2t, 2t+1 -> bins 2047-2t, 2046-2t (top first)
    const int t = threadIdx.x;
    const uint32_t c0 = sh.hist[kBins - 1 - 2 * t], c1 = sh.hist[kBins - 2 - 2 * t];
    const uint32_t ex = block_excl_scan(c0 + c1, sh);
    if (ex < (uint32_t)need && (uint32_t)need <= ex + c0) {
        sh.bin = kBins - 1 - 2 * t;
        sh.above = ex;
        sh.inbin = c0;
    } else if (ex + c0 < (uint32_t)need && (uint32_t)need <= ex + c0 + c1) {
        sh.bin = kBins - 2 - 2 * t;
        sh.above = ex + c0;
        sh.inbin = c1;
    }
    __syncthreads();
    const uint32_t bin = sh.bin, inbin = sh.inbin;
    need -= (int)sh.above;
    prefix |= (uint64_t)bin << sft;
    pmask |= (uint64_t)wm << sft;
    __syncthreads();
    return inbin;
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

struct LdsSrc {
    const uint64_t* c;
    int64_t count;
    __device__ __forceinline__ uint64_t get(int64_t e, bool& ok) const
    {
        ok = true;
        return c[e];
    }
};

// Exact need-th largest (1-based) of the unique composites of src: 11-bit
// radix levels over src until the bin that holds it fits in LDS, then the
// remaining levels over that LDS copy.
template <class Src>
__device__ uint64_t kth_largest(const Src& src, int need, SelShared& sh)
{
    uint64_t prefix = 0, pmask = 0;
    const int shifts[6] = {53, 42, 31, 20, 9, 0};
    int lvl = 0;
    uint32_t inbin = 0;
    for (; lvl < 6; ++lvl) {
        inbin = radix_level(src, shifts[lvl], lvl == 5 ? 0x1FFu : 0x7FFu, prefix, pmask, need, sh);
        if (inbin <= (uint32_t)kBuf) break;
    }
    // gather the bin into LDS
    if (threadIdx.x == 0) sh.nbuf = 0;
    __syncthreads();
    for (int64_t e = threadIdx.x; e < src.count; e += blockDim.x) {
        bool ok;
        const uint64_t v = src.get(e, ok);
        if (ok && (v & pmask) == prefix) {
            const uint32_t slot = atomicAdd(&sh.nbuf, 1u);
            if (slot < (uint32_t)kBuf) sh.buf[slot] = v;
        }
    }
    __syncthreads();
    const LdsSrc lsrc{sh.buf, (int64_t)(inbin < (uint32_t)kBuf ? inbin : kBuf)};
    for (++lvl; lvl < 6 && inbin > 1; ++lvl)
        inbin = radix_level(lsrc, shifts[lvl], lvl == 5 ? 0x1FFu : 0x7FFu, prefix, pmask, need, sh);
    // the single element with this prefix
    if (threadIdx.x == 0) sh.result = 0;
    __syncthreads();
    for (int64_t e = threadIdx.x; e < lsrc.count; e += blockDim.x)
        if ((sh.buf[e] & pmask) == prefix) sh.result = sh.buf[e];
    __syncthreads();
    const uint64_t T = sh.result;
    __syncthreads();
    return T;
}

__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t* p, int64_t cnt, uint32_t v)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < cnt) p[i] = v;
}

// flags[p] = 1 when some head of pair p collected more candidates than fit.
__global__ __launch_bounds__(256) void overflow_kernel(const uint32_t* __restrict__ counts, int P,
                                                       int G, int64_t cap, uint32_t* __restrict__ flags)
{
    const int p = blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= P) return;
    uint32_t f = 0;
    for (int h = 0; h < G; ++h) f |= (int64_t)counts[(size_t)p * G + h] > cap ? 1u : 0u;
    flags[p] = f;
}

__global__ __launch_bounds__(kSelThreads) void threshold_kernel(const float* __restrict__ scores,
                                                                int64_t n, int64_t npad,
                                                                int64_t stride, int64_t count,
                                                                int64_t valid, int k,
                                                                uint32_t* __restrict__ tau)
{
    __shared__ SelShared sh;
    const int64_t m = blockIdx.x;
    if (valid < k) {
        if (threadIdx.x == 0) tau[m] = 0u;
        return;
    }
    // Any lower bound of the k-th largest score is a valid threshold: two
    // 11-bit radix levels locate the bin (the top 22 bits of the key) that
    // holds the sample's k-th largest, and its lower edge is used -- within
    // 2^-14 of that value, and every element of the bin is at or above it.
    DenseSrc src{scores + m * npad, n, stride, count};
    uint64_t prefix = 0, pmask = 0;
    int need = k;
    radix_level(src, 53, 0x7FFu, prefix, pmask, need, sh);
    radix_level(src, 42, 0x7FFu, prefix, pmask, need, sh);
    if (threadIdx.x == 0) tau[m] = (uint32_t)(prefix >> 32);
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

__global__ __launch_bounds__(kSelThreads) void select_kernel(
    const float* __restrict__ scores, int64_t n, int64_t npad, const uint32_t* __restrict__ counts,
    const uint64_t* __restrict__ cand, int64_t cap, int k, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_val, int32_t* __restrict__ sorted_idx)
{
    __shared__ SelShared sh;
    const int64_t m = blockIdx.x;
    const int64_t cnt = counts[m];
    uint64_t T;
    const bool dense = cnt > cap;
    DenseSrc dsrc{scores + m * npad, n, 1, npad};
    CandSrc csrc{cand + m * cap, cnt};
    T = dense ? kth_largest(dsrc, k, sh) : kth_largest(csrc, k, sh);
    // gather the k winners (composites >= T); each one's rank among them is
    // its output position (composites are unique)
    if (threadIdx.x == 0) sh.nbuf = 0;
    __syncthreads();
    const int64_t total = dense ? dsrc.count : csrc.count;
    for (int64_t e = threadIdx.x; e < total; e += blockDim.x) {
        bool ok;
        const uint64_t v = dense ? dsrc.get(e, ok) : csrc.get(e, ok);
        if (ok && v >= T) {
            const uint32_t slot = atomicAdd(&sh.nbuf, 1u);
            if (slot < (uint32_t)kBuf) sh.buf[slot] = v;
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
            sh.hist[c * kWave + lane] = sl;
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
                const uint32_t lo = sh.hist[slot];
                sorted_idx[m * k + count_above(sh.hist, nch, lo)] = (int32_t)(~lo);
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
__global__ __launch_bounds__(kSelThreads) void union_kernel(const int32_t* __restrict__ sorted_idx,
                                                            int G, int k,
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
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const int e = threadIdx.x + u * (int)blockDim.x;
        pos[u] = -1;
        val[u] = 0;
        if (e < total) {
            const int h = e / k;
            const int32_t x = a[e];
            int r = e - h * k;
            for (int h2 = 0; h2 < G; ++h2) {
                if (h2 == h) continue;
                const int32_t* l = a + h2 * k;
                int lo = 0, hi = k;  // first element of list h2 placed after x
                while (lo < hi) {
                    const int mid = (lo + hi) >> 1;
                    const bool before = h2 < h ? l[mid] <= x : l[mid] < x;
                    if (before) lo = mid + 1;
                    else hi = mid;
                }
                r += lo;
            }
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
    uint32_t x = cnt;
    for (int o = 1; o < kWave; o <<= 1) {
        const uint32_t y = __shfl_up(x, o, kWave);
        if (lane >= o) x += y;
    }
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
    // per-lane maxima (one value per 32 or 16 tokens) carry almost the same
    // tail information as the tokens themselves once there are >= 4k of them
    L.lanemax = n >= 128 * (int64_t)k * s;
    L.cap = 8 * (int64_t)k * s + 1024;
    if (L.cap > nb * 64) L.cap = nb * 64;
    L.sample_nlb = ((nb + 32 * s - 1) / (32 * s)) * 32;
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    L.off_tau = 0;
    L.off_count = up((size_t)L.m * 4);
    L.off_cand = up(L.off_count + (size_t)L.m * 4);
    L.off_sorted = up(L.off_cand + (size_t)L.m * (size_t)L.cap * 8);
    L.bytes = L.off_sorted + (size_t)L.m * (size_t)k * 4;
    L.off_flags = up(L.bytes);
    L.off_sample = up(L.off_flags + (size_t)P * 4);
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

    fill_u32_kernel<<<dim3((unsigned)((L.m + 255) / 256)), 256, 0, st>>>(counts, L.m, 0u);
    threshold_kernel<<<dim3((unsigned)L.m), kSelThreads, 0, st>>>(scores, n, npad, L.stride,
                                                                 L.sample_nlb * 64, valid, k, tau);
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
    select_kernel<<<dim3((unsigned)L.m), kSelThreads, 0, st>>>(scores, n, npad, counts, cand, L.cap,
                                                              k, topk_idx, topk_val, sorted);
    union_kernel<<<dim3((unsigned)P), kSelThreads, 0, st>>>(sorted, G, k, union_idx, union_len);
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
    uint32_t* flags = (uint32_t*)(w + L.off_flags);
    float* sample = (float*)(w + L.off_sample);
    float* repair = (float*)(w + L.off_repair);
    hipError_t e;
    ScanArgs a = base;

    if (stages & 1) {
        // threshold: scores of every stride-th block, exact k-th largest
        fill_u32_kernel<<<dim3((unsigned)((L.m + 255) / 256)), 256, 0, st>>>(counts, L.m, 0u);
        a.stride = L.stride;
        a.nlb = L.sample_nlb;
        a.out = sample;
        a.only = nullptr;
        if ((e = launch_scan_args(a, P, G, L.lanemax ? 2 : 0, st)) != hipSuccess) return e;
        // every lane maximum is a distinct token's score, so the k-th largest
        // of them is still a lower bound of the k-th largest score
        const int64_t row = L.sample_nlb * (L.lanemax ? (G <= 4 ? 2 : 4) : 64);
        threshold_kernel<<<dim3((unsigned)L.m), kSelThreads, 0, st>>>(sample, row, row, 1, row, row,
                                                                     k, tau);
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
        a.only = nullptr;
        if ((e = launch_scan_args(a, P, G, 1, st)) != hipSuccess) return e;
    }
    if (stages & 4) {
        // pairs whose candidates overflowed get their full scores recomputed
        overflow_kernel<<<dim3((unsigned)((P + 255) / 256)), 256, 0, st>>>(counts, P, G, L.cap, flags);
        a = base;
        a.stride = 1;
        a.nlb = nb;
        a.out = repair;
        a.only = flags;
        if ((e = launch_scan_args(a, P, G, 0, st)) != hipSuccess) return e;
        // exact top-k of the candidates (or of the repaired scores), union
        int32_t* sorted = (int32_t*)(w + L.off_sorted);
        select_kernel<<<dim3((unsigned)L.m), kSelThreads, 0, st>>>(repair, n, npad, counts, cand,
                                                                  L.cap, k, topk_idx, topk_val, sorted);
        union_kernel<<<dim3((unsigned)P), kSelThreads, 0, st>>>(sorted, G, k, union_idx, union_len);
    }
    return hipGetLastError();
}

}  // namespace fathom

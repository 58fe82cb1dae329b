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
//                same select directly over all its scores instead: over the
//                given scores, or in the fused path over a full score row
//                its pair is rescanned into (a bounded number of rows in the
//                workspace: the first failed pairs rescanned by many
//                workgroups, any further ones by one workgroup per row).
//  4. union:     merge of the G index-sorted lists of a pair, duplicates
//                dropped.
#include "select.h"

namespace fathom {
namespace {

__global__ __launch_bounds__(kSelThreads) void threshold_kernel(const float* __restrict__ scores,
                                                                int64_t n, int64_t npad,
                                                                int64_t stride, int64_t count,
                                                                int64_t valid, int k,
                                                                uint32_t* __restrict__ tau,
                                                                uint32_t* __restrict__ counts)
{
    __shared__ SelSharedHist sh;
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

// A selection whose candidates overflowed their capacity, or number fewer
// than k, is selected over its full score row when `scores` is given (top-k
// of materialised scores); in the fused path (scores NULL) the repair
// kernel has selected it.  SH, NS and WPE (waves per SIMD the registers
// must allow) come in two forms: k <= 2048 with 8 register slots and the
// small buffer, four workgroups per CU (stage 3 at 1M tokens x 288 pairs
// 0.067 -> 0.063 ms); larger k with 16 slots and the full buffer, three.
template <class SH, int NS, int WPE>
__global__ __launch_bounds__(kSelectThreads, WPE) void select_kernel(
    const float* __restrict__ scores, int64_t n, int64_t npad, const uint32_t* __restrict__ counts,
    const uint64_t* __restrict__ cand, int64_t cap, int k, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_val, int32_t* __restrict__ sorted_idx)
{
    __shared__ SH sh;
    const int64_t m = blockIdx.x;
    const int64_t cnt = counts[m];
    const bool dense = cnt > cap || cnt < (int64_t)k;
    if (dense && !scores) return;
    select_one<NS>(dense ? scores + m * npad : nullptr, n, npad, dense, cand + m * cap, cnt, k, m, topk_idx,
                   topk_val, sorted_idx, sh);
}

// Union of the G winner lists of a pair, each sorted by token index: every
// element's place in the merged order is its own position plus the number
// of elements of each other list that precede it (binary search; equal
// indices ordered by list), then adjacent duplicates are dropped.  NPER:
// elements per thread, 2 when G k <= 2 blockDim (the code for more elements
// costs time even where it is not run), else kMaxUnion / kSelThreads.
template <int G, int NPER>
__global__ __launch_bounds__(kSelThreads) void union_kernel(const int32_t* __restrict__ sorted_idx,
                                                            int k,
                                                            int32_t* __restrict__ union_idx,
                                                            int32_t* __restrict__ union_len)
{
    constexpr int kPer = NPER;
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
        pos[u] = -1;
        val[u] = 0;
    }
    // binary lifting over each other list, steps from the largest power of
    // two not above k.  A thread's first two elements are searched together,
    // their 2 (G - 1) searches interleaved step by step (stage 3 at 1M x 288
    // pairs: 0.061 -> 0.058 ms); any further elements one at a time.
    const int top = 1 << (31 - __clz(k));
    {
        int own[2], sc[2][G];
        int32_t x[2];
#pragma unroll
        for (int v = 0; v < 2; ++v) {
            const int e = threadIdx.x + v * (int)blockDim.x;
            own[v] = e < total ? e / k : -1;
            x[v] = e < total ? a[e] : 0;
#pragma unroll
            for (int h2 = 0; h2 < G; ++h2) sc[v][h2] = 0;
        }
        for (int st = top; st > 0; st >>= 1) {
#pragma unroll
            for (int v = 0; v < 2; ++v)
#pragma unroll
                for (int h2 = 0; h2 < G; ++h2) {
                    const int np = sc[v][h2] + st;
                    if (own[v] >= 0 && h2 != own[v] && np <= k) {
                        const int32_t y = a[h2 * k + np - 1];
                        if (h2 < own[v] ? y <= x[v] : y < x[v]) sc[v][h2] = np;
                    }
                }
        }
#pragma unroll
        for (int v = 0; v < 2; ++v) {
            if (own[v] < 0) continue;
            int r = threadIdx.x + v * (int)blockDim.x - own[v] * k;
#pragma unroll
            for (int h2 = 0; h2 < G; ++h2) r += h2 != own[v] ? sc[v][h2] : 0;
            val[v] = x[v];
            pos[v] = r;
        }
    }
#pragma unroll
    for (int u = 2; u < kPer; ++u) {
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
template <int G>
void launch_union_g(const int32_t* sorted, int P, int k, int32_t* union_idx, int32_t* union_len, hipStream_t st)
{
    const dim3 grid((unsigned)P);
    if (G * k <= 2 * kSelThreads)
        union_kernel<G, 2><<<grid, kSelThreads, 0, st>>>(sorted, k, union_idx, union_len);
    else
        union_kernel<G, kMaxUnion / kSelThreads><<<grid, kSelThreads, 0, st>>>(sorted, k, union_idx, union_len);
}

void launch_union(const int32_t* sorted, int P, int G, int k, int32_t* union_idx, int32_t* union_len,
                  hipStream_t st)
{
    switch (G) {
    case 1: launch_union_g<1>(sorted, P, k, union_idx, union_len, st); break;
    case 2: launch_union_g<2>(sorted, P, k, union_idx, union_len, st); break;
    case 3: launch_union_g<3>(sorted, P, k, union_idx, union_len, st); break;
    case 4: launch_union_g<4>(sorted, P, k, union_idx, union_len, st); break;
    case 5: launch_union_g<5>(sorted, P, k, union_idx, union_len, st); break;
    case 6: launch_union_g<6>(sorted, P, k, union_idx, union_len, st); break;
    case 7: launch_union_g<7>(sorted, P, k, union_idx, union_len, st); break;
    default: launch_union_g<8>(sorted, P, k, union_idx, union_len, st); break;
    }
}

void launch_select(const float* scores, int64_t n, int64_t npad, const uint32_t* counts,
                   const uint64_t* cand, int64_t cap, int k, int32_t* topk_idx, float* topk_val,
                   int32_t* sorted, int64_t m, hipStream_t st)
{
    if (k <= SelSharedSmall::kCap)
        select_kernel<SelSharedSmall, 8, 8><<<dim3((unsigned)m), kSelectThreads, 0, st>>>(
            scores, n, npad, counts, cand, cap, k, topk_idx, topk_val, sorted);
    else
        select_kernel<SelShared, 16, 6><<<dim3((unsigned)m), kSelectThreads, 0, st>>>(
            scores, n, npad, counts, cand, cap, k, topk_idx, topk_val, sorted);
}

}  // namespace

// Over the host link the sample takes runs of 512 blocks (4 KB of each
// plane row): at 1M tokens x 288 pairs the step is 51.8-52.1 ms against
// 52.5 with runs of 32 (sample 3.67-3.83 against 3.97 ms, and the filter,
// which skips the sampled runs, reads fewer, longer pieces).
constexpr int kHostRunLog2 = 9;

TopkLayout topk_layout(int P, int G, int64_t n, int k, int rows, bool staged)
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
    L.staged = staged && s >= 2;
    L.lanemax = n >= 128 * (int64_t)k * s;
    // the fused threshold is the rank-th largest sample value: with one run
    // in every s sampled, about rank * s >= 2k scores lie above it.  That is
    // a statistical bound; a selection that ends up with fewer than k
    // candidates is selected over all of its scores instead (stage 3).
    L.rank = s == 1 ? k : (int)((2 * (int64_t)k + s - 1) / s);
    L.cap = 8 * (int64_t)k * s + 1024;
    if (L.cap > nb * 64) L.cap = nb * 64;
    // runs of 32 blocks; over the host link runs of 512
    L.run_log2 = L.staged ? kHostRunLog2 : 5;
    const int64_t run = (int64_t)1 << L.run_log2;
    L.sample_nlb = ((nb + run * s - 1) / (run * s)) * run;
    L.slots = P < rows ? P : rows;
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    L.off_tau = 0;
    L.off_count = up((size_t)L.m * 4);
    L.off_cand = up(L.off_count + (size_t)L.m * 4);
    L.off_sorted = up(L.off_cand + (size_t)L.m * (size_t)L.cap * 8);
    L.bytes = L.off_sorted + (size_t)L.m * (size_t)k * 4;
    // the sample: per-lane maxima (4 per block) or every score (64 per block)
    L.off_sample = up(L.bytes);
    L.off_repair = L.off_sample;
    size_t sample_bytes = (size_t)L.m * (size_t)L.sample_nlb * (L.lanemax ? 4 : 64) * 4;
    L.off_scores = L.off_sample;
    if (L.staged && L.lanemax) {  // the maxima set the threshold; every score is kept beside them
        L.off_scores = up(L.off_sample + sample_bytes);
        sample_bytes = L.off_scores - L.off_sample + (size_t)L.m * (size_t)L.sample_nlb * 64 * 4;
    }
    const size_t repair_bytes = (size_t)L.slots * (size_t)G * (size_t)nb * 64 * 4;
    L.bytes_fused = L.off_sample + (sample_bytes > repair_bytes ? sample_bytes : repair_bytes);
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
    launch_select(scores, n, npad, counts, cand, L.cap, k, topk_idx, topk_val, sorted, L.m, st);
    launch_union(sorted, P, G, k, union_idx, union_len, st);
    return hipGetLastError();
}

// Fused path, stage 2, staged sample: the scores that stage 1 stored for
// the sampled runs (row m: [sample_nlb * 64], tokens past n and blocks past
// the index at -inf) are kept where they reach their selection's threshold,
// as the filtered scan keeps its own candidates (same keys, same capacity
// rule).  Grid: (selection m, chunks of its row).
__global__ __launch_bounds__(256) void sample_filter_kernel(const float* __restrict__ sample, int64_t row,
                                                            int64_t n, int64_t stride, int rl,
                                                            const uint32_t* __restrict__ tau,
                                                            uint32_t* __restrict__ counts,
                                                            uint64_t* __restrict__ cand, int64_t cap)
{
    const int64_t m = blockIdx.x;
    const uint32_t tk = tau[m];
    const float th = tk <= 0x007FFFFFu ? -INFINITY : key_score(tk);
    const float* r = sample + m * row;
    const int lane = lane_id();
    for (int64_t e0 = (int64_t)blockIdx.y * blockDim.x; e0 < row; e0 += (int64_t)gridDim.y * blockDim.x) {
        const int64_t e = e0 + threadIdx.x;
        bool keep = false;
        float sc = 0.0f;
        int64_t tok = 0;
        if (e < row) {
            const int64_t lb = e >> 6;  // logical sample block: run lb >> rl, one in every stride
            tok = (((lb >> rl) * stride << rl) + (lb & (((int64_t)1 << rl) - 1))) * 64 + (e & 63);
            sc = r[e];
            keep = tok < n && sc >= th;
        }
        const uint64_t b = __ballot(keep);
        if (!b) continue;
        uint32_t base = 0;
        if (lane == 0) base = atomicAdd(&counts[m], (uint32_t)__popcll(b));
        base = (uint32_t)__shfl((int)base, 0, kWave);
        const uint32_t pos = base + (uint32_t)__popcll(b & lanes_below(lane));
        if (keep && (int64_t)pos < cap) cand[m * cap + pos] = composite(score_key(sc), (uint32_t)tok);
    }
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
    float* sample = (float*)(w + L.off_sample);
    float* repair = (float*)(w + L.off_repair);
    hipError_t e;
    ScanArgs a = base;

    if (stages & 1) {
        // threshold: scores of every stride-th block, exact k-th largest (the
        // threshold kernel also clears the candidate counts).  Staged, the
        // sample keeps every score it computes for stage 2.
        a.stride = L.stride;
        a.run_log2 = L.run_log2;
        a.nlb = L.sample_nlb;
        a.out = sample;
        a.out2 = L.staged && L.lanemax ? (float*)(w + L.off_scores) : nullptr;
        if ((e = launch_scan_args(a, P, G, L.lanemax ? 2 : 0, st)) != hipSuccess) return e;
        // every lane maximum is a distinct token's score, so the k-th largest
        // of them is still a lower bound of the k-th largest score
        const int64_t row = L.sample_nlb * (L.lanemax ? 4 : 64);
        threshold_kernel<<<dim3((unsigned)L.m), kSelectThreads, 0, st>>>(sample, row, row, 1, row, row,
                                                                     L.rank, tau, counts);
    }
    if (stages & 2) {
        // filter: every block, keeping the scores at or above the threshold.
        // Staged, the sampled runs are not read again: their stored scores
        // are filtered instead, so every index byte crosses the link once.
        a = base;
        a.stride = 1;
        a.skip = L.staged ? L.stride : 0;
        a.run_log2 = L.run_log2;
        a.nlb = nb;
        a.tau = tau;
        a.counts = counts;
        a.cand = cand;
        a.cap = L.cap;
        if ((e = launch_scan_args(a, P, G, 1, st)) != hipSuccess) return e;
        if (L.staged) {
            const int64_t row = L.sample_nlb * 64;
            const int64_t chunks = (row + 4095) / 4096;  // 16 scores per thread
            sample_filter_kernel<<<dim3((unsigned)L.m, (unsigned)(chunks < 65535 ? chunks : 65535)), 256, 0, st>>>(
                (const float*)(w + L.off_scores), row, n, L.stride, L.run_log2, tau, counts, cand, L.cap);
        }
    }
    if (stages & 4) {
        // selections whose candidates failed (overflow, or fewer than k):
        // their pairs rescanned into the repair rows and selected there;
        // the others from their candidates; then the union
        int32_t* sorted = (int32_t*)(w + L.off_sorted);
        if ((e = launch_repair(base, P, G, k, counts, L.cap, repair, L.slots, topk_idx, topk_val, sorted,
                               st)) != hipSuccess)
            return e;
        launch_select(nullptr, n, npad, counts, cand, L.cap, k, topk_idx, topk_val, sorted, L.m, st);
        launch_union(sorted, P, G, k, union_idx, union_len, st);
    }
    return hipGetLastError();
}

}  // namespace fathom

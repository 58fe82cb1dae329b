// Internal helpers shared by the gfx950 kernels of the Fathom key scan.
// Not part of the public ABI (that is include/fathom.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fathom {

constexpr int kWave = 64;
constexpr int kMaxD = 128;
constexpr int kMaxG = 8;
constexpr int kMaxK = 4096;
constexpr int kMaxPairs = 65535;  // P per call: pairs run on grid.y
constexpr int kMaxUnion = 16384;  // G * k handled by the union kernel

// ---------------------------------------------------------------- numerics

// IEEE binary16 -> float32 (exact), from the bit fields.
__device__ __forceinline__ float f16_bits_to_f32(uint32_t h)
{
    uint32_t ex = (h >> 10) & 31u, man = h & 1023u, sign = (h & 0x8000u) << 16;
    uint32_t bits;
    if (ex == 0) {
        float v = (float)man * 5.9604644775390625e-8f;  // man * 2^-24, exact
        return (h & 0x8000u) ? -v : v;
    }
    if (ex == 31) bits = sign | 0x7F800000u | (man << 13);
    else bits = sign | ((ex + 112u) << 23) | (man << 13);
    return __uint_as_float(bits);
}

// Non-negative finite float32 -> binary16, round to nearest even, with
// values at or above 65520 (which would round to infinity) saturated to 65504.
__device__ __forceinline__ uint32_t f32_to_f16_rne_sat(float m)
{
    uint32_t u = __float_as_uint(m) & 0x7FFFFFFFu;
    if (u >= 0x477FF000u) return 0x7BFFu;
    int e = (int)(u >> 23) - 127;
    uint32_t mant = u & 0x7FFFFFu;
    if (e >= -14) {
        uint32_t h = ((uint32_t)(e + 15) << 10) | (mant >> 13);
        uint32_t rem = mant & 0x1FFFu;
        if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h += 1u;
        return h;
    }
    if (e < -25) return 0u;
    uint32_t m24 = mant | 0x800000u;
    int sh = -1 - e;  // 14 .. 24
    uint32_t h = m24 >> sh;
    uint32_t rem = m24 & ((1u << sh) - 1u);
    uint32_t half = 1u << (sh - 1);
    if (rem > half || (rem == half && (h & 1u))) h += 1u;
    return h;
}

// Order-preserving map of a score to uint32 (ascending key = ascending
// score); -0 is folded onto +0 so that the two compare equal.
__device__ __forceinline__ uint32_t score_key(float s)
{
    uint32_t u = __float_as_uint(s == 0.0f ? 0.0f : s);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_score(uint32_t k)
{
    uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(u);
}

// Composite sort key: descending order = score descending, index ascending.
__device__ __forceinline__ uint64_t composite(uint32_t key, uint32_t idx)
{
    return ((uint64_t)key << 32) | (uint64_t)(~idx);
}

// ------------------------------------------------------------ wave helpers

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

__device__ __forceinline__ uint64_t lanes_below(int lane)
{
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

__device__ __forceinline__ int wave_sum_i32(int v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ __forceinline__ float wave_max_f32(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

// --------------------------------------------------------- host launchers

// Packs tokens [tok0, tok0 + m) of every pair (tok0 a multiple of 64) into an
// index whose channel rows hold ldb blocks.
hipError_t launch_pack(const void* keys, int dtype, int P, int64_t tok0, int64_t m, int D,
                       const float* rot, uint64_t* planes, uint16_t* scales, int64_t ldb,
                       hipStream_t st);
hipError_t launch_plan(const float* q, const float* sigma2, const float* rot, int P, int G, int D,
                       int budget, int mode, uint8_t* depth, int16_t* active, int32_t* n_active,
                       float* theta, float* q_used, hipStream_t st);
hipError_t launch_scan(const uint64_t* planes, const uint16_t* scales, int P, int D, int64_t n,
                       int64_t ldb, const uint8_t* depth, const int16_t* active,
                       const int32_t* n_active, const float* q_used, int G, float* scores,
                       hipStream_t st);

// Arguments of the scan kernels (see scan.hip).
struct ScanArgs {
    const uint64_t* planes;
    const uint16_t* scales;
    int D;
    int64_t n, nb;         // tokens, and the blocks that hold them
    int64_t ldb;           // blocks per channel row of the index (>= nb)
    const uint8_t* depth;
    const int16_t* active;
    const int32_t* n_active;
    const float* q_used;
    int64_t stride;        // 1, or: scan one run of 32 consecutive blocks in every stride runs
    int64_t skip;          // 0, or a power of two s >= 2: the runs the sample took (one in every s,
                           // the first included) are neither read nor filtered
    int run_log2;          // sampled runs are 2^run_log2 blocks long (0: 32 blocks)
    int64_t nlb;           // logical blocks per pair (rows of the STORE output / 64)
    float* out;            // STORE: [P][G][nlb * 64]; LANEMAX: [P][G][nlb * 4] (maxima of 16 tokens)
    float* out2;           // LANEMAX, or null: every score as well ([P][G][nlb * 64], as STORE)
    const uint32_t* tau;   // FILTER: [P][G] key thresholds
    uint32_t* counts;      // FILTER: [P][G]
    uint64_t* cand;        // FILTER: [P][G][cap]
    int64_t cap;
    int gb;                // logical blocks per workgroup (set by the launcher)
};
// mode: 0 store scores, 1 filter into candidates, 2 per-lane maxima
hipError_t launch_scan_args(const ScanArgs& a, int P, int G, int mode, hipStream_t st);

hipError_t launch_gather(const void* table, int64_t table_rows, int64_t row_bytes,
                         int64_t pair_stride, int P, const int32_t* idx, const int32_t* len,
                         int cap, void* out, hipStream_t st);
hipError_t launch_read_probe(const void* src, size_t bytes, uint32_t* sink, hipStream_t st);

size_t calib_workspace_bytes(int P, int64_t m, int D);
hipError_t launch_calib_covariance(const void* keys, int dtype, int P, int64_t m, int D, double* cov,
                                   float* var, void* ws, hipStream_t st);
hipError_t launch_calib_basis(const double* cov, int P, int D, float* U, float* lam, hipStream_t st);

// Repair rows of the fused path: a workgroup per row rescans one failed pair
// at a time, so this bounds both the workspace and the repair's parallelism.
constexpr int kRepairSlots = 16;

struct TopkLayout {
    int64_t m;           // selections = P * G
    int64_t stride;      // sample one run of 32 blocks in every `stride` runs
    int64_t sample_nlb;  // logical sample blocks per pair (whole runs)
    int64_t cap;         // candidate capacity per selection
    bool lanemax;        // fused threshold from per-lane maxima of the sample
    bool staged;         // fused: the sample stores every score it reads, and stage 2 filters
                         // those stored scores instead of reading the sampled runs again
    int run_log2;        // the sample's runs are 2^run_log2 blocks long
    int rank;            // fused threshold: this order statistic of the sample
    size_t off_tau, off_count, off_cand, off_sorted, bytes;  // top-k from given scores
    int slots;           // fused: full score rows (pairs) for the repair, reused in turn
    size_t off_scores;   // staged: the sample's scores (the sample itself when it holds every score)
    size_t off_sample, off_repair, bytes_fused;  // fused scan + top-k (the sample, used by
                                                 // stages 1-2, and the repair rows, used by
                                                 // stage 3, share their memory)
};
// rows: repair rows of the fused path, at most this many (and at most P);
// staged: the layout for an index the scan reads over the host link (taken
// only when the sample stride is at least 2)
TopkLayout topk_layout(int P, int G, int64_t n, int k, int rows = kRepairSlots, bool staged = false);
hipError_t launch_topk(const float* scores, int P, int G, int64_t n, int k, int32_t* topk_idx,
                       float* topk_val, int32_t* union_idx, int32_t* union_len, void* ws,
                       const TopkLayout& L, hipStream_t st);
// Selections whose candidate count c fails (c > cap or c < k): each of
// `slots` workgroups rescans failed pairs in turn into its own row of
// G x npad scores (rows: [slots][G][npad] floats) and selects the failed
// heads there exactly.
hipError_t launch_repair(const ScanArgs& base, int P, int G, int k, const uint32_t* counts, int64_t cap,
                         float* rows, int slots, int32_t* topk_idx, float* topk_val, int32_t* sorted_idx,
                         hipStream_t st);
hipError_t launch_scan_topk(const ScanArgs& base, int P, int G, int k, int32_t* topk_idx,
                            float* topk_val, int32_t* union_idx, int32_t* union_len, void* ws,
                            const TopkLayout& L, int stages, hipStream_t st);

}  // namespace fathom

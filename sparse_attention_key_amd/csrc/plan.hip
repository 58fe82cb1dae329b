// Per-pair read plan (yeyulingfeng.com write-up of Fathom, section "方法二":
// importance = calibration variance times the group's query energy, integer
// reverse water-filling with one water level per query group, channels at or
// below the level skipped; section "基座选择": queries rotated into the
// stored basis).
//
// One wavefront per pair; lane l owns channels l and l + 64.  The level is
// found by bisection over the float32 bit patterns of theta (monotone for
// theta >= 0): 31 steps, each an exact count of sum_j t_j(theta) reduced
// across the wavefront, so the result is the exact smallest feasible level
// with no transcendental functions involved.
#include "common.h"

namespace fathom {
namespace {

__device__ __forceinline__ int depth_at(float w, float theta)
{
    int t = 0;
    float lvl = theta;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        t += (w > lvl) ? 1 : 0;
        lvl = lvl * 4.0f;
    }
    return t;
}

// Sum of depths over the wavefront's channels at level theta.  A lane's
// share is 0..8, so the sum is assembled from one wavefront mask per bit
// (four ballots and population counts instead of a shuffle chain).
__device__ __forceinline__ int total_depth(float w0, float w1, bool has0, bool has1, float theta)
{
    const int s = (has0 ? depth_at(w0, theta) : 0) + (has1 ? depth_at(w1, theta) : 0);
    int t = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) t += __popcll(__ballot((s >> b) & 1)) << b;
    return t;
}

// Fixed r-channel plan: rank by group query energy, ties to the lower channel.
__device__ int topr_depth(const float* s_sq, int D, float sq, int j, int r)
{
    int rank = 0;
    for (int i = 0; i < D; ++i) rank += (s_sq[i] > sq || (s_sq[i] == sq && i < j)) ? 1 : 0;
    return rank < r ? 4 : 0;
}

__global__ __launch_bounds__(64) void plan_kernel(const float* __restrict__ q,
                                                  const float* __restrict__ sigma2,
                                                  const float* __restrict__ rot, int G, int D,
                                                  int budget, int mode,
                                                  uint8_t* __restrict__ depth,
                                                  int16_t* __restrict__ active,
                                                  int32_t* __restrict__ n_active,
                                                  float* __restrict__ theta_out,
                                                  float* __restrict__ q_used)
{
    __shared__ float s_q[kMaxG][kMaxD];
    __shared__ float s_sq[kMaxD];
    const int p = blockIdx.x, lane = lane_id();
    // every query value and variance the lane needs is requested at once (a
    // lane past D reads channel D - 1, a head past G head G - 1, and drops
    // them), so the kernel waits for one round trip to memory
    int jc[2];
    float qv[2][kMaxG], sg[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int j = lane + c * kWave;
        jc[c] = j < D ? j : D - 1;
#pragma unroll
        for (int h = 0; h < kMaxG; ++h)
            qv[c][h] = q[((size_t)p * G + (h < G ? h : G - 1)) * D + jc[c]];
        sg[c] = sigma2[(size_t)p * D + jc[c]];
    }
    if (rot) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
            if (lane + c * kWave < D)
#pragma unroll
                for (int h = 0; h < kMaxG; ++h)
                    if (h < G) s_q[h][lane + c * kWave] = qv[c][h];
        __syncthreads();
        const float* U = rot + (size_t)p * D * D;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            if (lane + c * kWave >= D) continue;
#pragma unroll
            for (int h = 0; h < kMaxG; ++h) {
                if (h >= G) break;
                float acc = 0.0f;
                for (int d = 0; d < D; ++d) acc = __builtin_fmaf(U[(size_t)d * D + jc[c]], s_q[h][d], acc);
                qv[c][h] = acc;
            }
        }
    }

    float w[2] = {0.0f, 0.0f}, sq[2] = {0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int j = lane + c * kWave;
        if (j >= D) continue;
        float acc_sq = 0.0f;
#pragma unroll
        for (int h = 0; h < kMaxG; ++h) {
            if (h >= G) break;
            q_used[((size_t)p * G + h) * D + j] = qv[c][h];
            acc_sq = __builtin_fmaf(qv[c][h], qv[c][h], acc_sq);
        }
        sq[c] = acc_sq;
        const float v = sg[c] * acc_sq;
        w[c] = (v > 0.0f) ? v : 0.0f;
        s_sq[j] = acc_sq;
    }
    __syncthreads();

    const bool has0 = lane < D, has1 = lane + kWave < D;
    int t0 = 0, t1 = 0;
    float theta = 0.0f;
    if (mode == 2) {
        t0 = budget;
        t1 = budget;
    } else if (mode == 1) {
        t0 = has0 ? topr_depth(s_sq, D, sq[0], lane, budget) : 0;
        t1 = has1 ? topr_depth(s_sq, D, sq[1], lane + kWave, budget) : 0;
    } else {
        if (total_depth(w[0], w[1], has0, has1, 0.0f) > budget) {
            uint32_t lo = 0u, hi = 0x7F800000u;  // total(lo) > budget >= total(hi)
            while (hi - lo > 1u) {
                const uint32_t mid = lo + ((hi - lo) >> 1);
                if (total_depth(w[0], w[1], has0, has1, __uint_as_float(mid)) <= budget) hi = mid;
                else lo = mid;
            }
            theta = __uint_as_float(hi);
        }
        t0 = depth_at(w[0], theta);
        t1 = depth_at(w[1], theta);
    }
    if (!has0) t0 = 0;
    if (!has1) t1 = 0;

    const uint64_t m0 = __ballot(t0 > 0), m1 = __ballot(t1 > 0);
    const uint64_t below = lanes_below(lane);
    const int na = __popcll(m0) + __popcll(m1);
    int16_t* act = active + (size_t)p * D;
    if (t0 > 0) act[__popcll(m0 & below)] = (int16_t)lane;
    if (t1 > 0) act[__popcll(m0) + __popcll(m1 & below)] = (int16_t)(lane + kWave);
    for (int e = na + lane; e < D; e += kWave) act[e] = -1;
    if (lane < D) depth[(size_t)p * D + lane] = (uint8_t)t0;
    if (lane + kWave < D) depth[(size_t)p * D + lane + kWave] = (uint8_t)t1;
    if (lane == 0) {
        n_active[p] = na;
        theta_out[p] = theta;
    }
}

}  // namespace

hipError_t launch_plan(const float* q, const float* sigma2, const float* rot, int P, int G, int D,
                       int budget, int mode, uint8_t* depth, int16_t* active, int32_t* n_active,
                       float* theta, float* q_used, hipStream_t st)
{
    plan_kernel<<<dim3((unsigned)P), 64, 0, st>>>(q, sigma2, rot, G, D, budget, mode, depth, active,
                                                  n_active, theta, q_used);
    return hipGetLastError();
}

}  // namespace fathom

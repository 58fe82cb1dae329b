// Approximate scores of every key from the bit-plane index (yeyulingfeng.com
// write-up of Fathom: section "方法一" -- a t-plane prefix is the t-bit
// mid-rise quantiser; section "方法二" -- only the first t_j planes of each
// active channel are read, and the plan is shared by the G heads of a group
// so the index is read once for all of them).
//
// Score contract: for token i and head h, s = 0 and for each active channel
// j in ascending order s = fma(q_hj, khat_ij, s), with khat_ij the exact
// dequantised prefix (2 c_t + 1 - 2^t) * 2^-t * scale.
//
// Simple form: one wavefront per 64-token block, lane i = token i, so every
// plane word is wavefront-uniform; G float32 accumulators per lane.
#include "common.h"

namespace fathom {
namespace {

template <int G>
__global__ __launch_bounds__(256) void scan_block_kernel(
    const uint64_t* __restrict__ planes, const uint16_t* __restrict__ scales, int D, int64_t n,
    int64_t nb, const uint8_t* __restrict__ depth, const int16_t* __restrict__ active,
    const int32_t* __restrict__ n_active, const float* __restrict__ q_used,
    float* __restrict__ scores)
{
    __shared__ float s_q[kMaxD][G];
    __shared__ int s_j[kMaxD];
    __shared__ int s_t[kMaxD];
    const int p = blockIdx.y;
    const int A = n_active[p];
    for (int a = threadIdx.x; a < A; a += blockDim.x) {
        const int j = active[(size_t)p * D + a];
        s_j[a] = j;
        s_t[a] = depth[(size_t)p * D + j];
#pragma unroll
        for (int h = 0; h < G; ++h) s_q[a][h] = q_used[((size_t)p * G + h) * D + j];
    }
    __syncthreads();

    const int wave = threadIdx.x / kWave, lane = lane_id();
    const int64_t b = (int64_t)blockIdx.x * 4 + wave;
    if (b >= nb) return;
    const uint64_t* pl = planes + (size_t)p * D * 4 * nb + b;
    const uint16_t* sc = scales + (size_t)p * D * nb + b;

    float acc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) acc[h] = 0.0f;
    for (int a = 0; a < A; ++a) {
        const int j = s_j[a], t = s_t[a];
        const uint64_t* wj = pl + (size_t)j * 4 * nb;
        uint32_t c = 0;
        for (int s = 0; s < t; ++s) c = (c << 1) | (uint32_t)((wj[(size_t)s * nb] >> lane) & 1ull);
        const float step = f16_bits_to_f32(sc[(size_t)j * nb]) * __uint_as_float((uint32_t)(127 - t) << 23);
        const float kh = (float)((int)(2u * c + 1u) - (1 << t)) * step;
#pragma unroll
        for (int h = 0; h < G; ++h) acc[h] = __builtin_fmaf(s_q[a][h], kh, acc[h]);
    }
    const int64_t tok = b * 64 + lane;
    const int64_t npad = nb * 64;
#pragma unroll
    for (int h = 0; h < G; ++h)
        scores[((size_t)p * G + h) * npad + tok] = tok < n ? acc[h] : -INFINITY;
}

template <int G>
hipError_t launch_g(const uint64_t* planes, const uint16_t* scales, int P, int D, int64_t n,
                    const uint8_t* depth, const int16_t* active, const int32_t* n_active,
                    const float* q_used, float* scores, hipStream_t st)
{
    const int64_t nb = (n + 63) / 64;
    dim3 grid((unsigned)((nb + 3) / 4), (unsigned)P);
    scan_block_kernel<G><<<grid, 256, 0, st>>>(planes, scales, D, n, nb, depth, active, n_active,
                                               q_used, scores);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_scan(const uint64_t* planes, const uint16_t* scales, int P, int D, int64_t n,
                       const uint8_t* depth, const int16_t* active, const int32_t* n_active,
                       const float* q_used, int G, float* scores, hipStream_t st)
{
    switch (G) {
    case 1: return launch_g<1>(planes, scales, P, D, n, depth, active, n_active, q_used, scores, st);
    case 2: return launch_g<2>(planes, scales, P, D, n, depth, active, n_active, q_used, scores, st);
    case 3: return launch_g<3>(planes, scales, P, D, n, depth, active, n_active, q_used, scores, st);
    case 4: return launch_g<4>(planes, scales, P, D, n, depth, active, n_active, q_used, scores, st);
    case 5: return launch_g<5>(planes, scales, P, D, n, depth, active, n_active, q_used, scores, st);
    case 6: return launch_g<6>(planes, scales, P, D, n, depth, active, n_active, q_used, scores, st);
    case 7: return launch_g<7>(planes, scales, P, D, n, depth, active, n_active, q_used, scores, st);
    default: return launch_g<8>(planes, scales, P, D, n, depth, active, n_active, q_used, scores, st);
    }
}

}  // namespace fathom

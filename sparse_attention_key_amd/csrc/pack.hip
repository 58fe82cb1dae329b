// Quantise keys into the channel-major bit-plane index (yeyulingfeng.com
// write-up of Fathom, section "方法一": per-channel uniform symmetric 4-bit
// code, one fp16 scale per 64-token block, bit p of the block's 64 codes in
// one 64-bit plane word, planes laid out along the sequence per channel).
//
// One workgroup (4 wavefronts) packs 16 consecutive blocks of one pair.  A
// wavefront owns one block at a time with lane i = token i, so the block max
// is a wavefront max-reduction and each plane word is one ballot.  Words are
// collected in LDS as [channel][plane][16 blocks] and written out as whole
// 128-byte rows, so the scattered per-block words never hit HBM one by one.
#include "common.h"

namespace fathom {
namespace {

constexpr int kRun = 16;  // blocks per workgroup

// Exact floor(x / delta) + 8, clamped to the 4-bit range.  delta = scale/8
// has at most 11 significant bits and |x / delta| stays below ~9 inside a
// block, so f * delta is exact and two comparisons repair the rounding of
// x * (1/delta).
__device__ __forceinline__ uint32_t quant_code(float x, float delta, float inv)
{
    if (!(delta > 0.0f)) return 8u;
    float f = floorf(x * inv);
    if (f * delta > x) f -= 1.0f;
    else if ((f + 1.0f) * delta <= x) f += 1.0f;
    f = fminf(fmaxf(f + 8.0f, 0.0f), 15.0f);
    return (uint32_t)f;
}

template <int DTYPE>
__device__ __forceinline__ float load_key(const void* keys, size_t off)
{
    if (DTYPE == 0) return ((const float*)keys)[off];
    uint32_t b = ((const uint16_t*)keys)[off];
    return __uint_as_float(b << 16);  // bfloat16 widens exactly
}

template <int DTYPE, bool ROT>
__global__ __launch_bounds__(256) void pack_kernel(const void* __restrict__ keys, int64_t n,
                                                   int D, int64_t nb,
                                                   const float* __restrict__ rot,
                                                   uint64_t* __restrict__ planes,
                                                   uint16_t* __restrict__ scales)
{
    __shared__ uint64_t s_words[kMaxD * 4 * kRun];  // 64 KB
    __shared__ uint16_t s_scale[kMaxD * kRun];

    const int p = blockIdx.y;
    const int64_t b0 = (int64_t)blockIdx.x * kRun;
    const int wave = threadIdx.x / kWave, lane = lane_id();
    const float* U = ROT ? rot + (size_t)p * D * D : nullptr;

    for (int r = wave; r < kRun; r += 4) {
        const int64_t b = b0 + r;
        if (b >= nb) break;
        const int64_t tok = b * 64 + lane;
        const bool valid = tok < n;
        const size_t row = ((size_t)p * n + (size_t)(valid ? tok : 0)) * D;
        for (int j = 0; j < D; ++j) {
            float x;
            if (ROT) {
                float acc = 0.0f;
                for (int d = 0; d < D; ++d)
                    acc = __builtin_fmaf(U[(size_t)d * D + j], load_key<DTYPE>(keys, row + d), acc);
                x = acc;
            } else {
                x = load_key<DTYPE>(keys, row + j);
            }
            const float m = wave_max_f32(valid ? fabsf(x) : 0.0f);
            const uint32_t sb = f32_to_f16_rne_sat(m);
            const float delta = f16_bits_to_f32(sb) * 0.125f;
            const float inv = 1.0f / delta;
            const uint32_t c = valid ? quant_code(x, delta, inv) : 8u;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const uint64_t word = __ballot((c >> (3 - s)) & 1u);
                if (lane == 0) s_words[(j * 4 + s) * kRun + r] = word;
            }
            if (lane == 0) s_scale[j * kRun + r] = (uint16_t)sb;
        }
    }
    __syncthreads();

    const int runs = (int)((nb - b0) < kRun ? (nb - b0) : kRun);
    for (int e = threadIdx.x; e < D * 4 * kRun; e += blockDim.x) {
        const int r = e % kRun, js = e / kRun;
        if (r < runs) planes[((size_t)p * D * 4 + js) * nb + b0 + r] = s_words[e];
    }
    for (int e = threadIdx.x; e < D * kRun; e += blockDim.x) {
        const int r = e % kRun, j = e / kRun;
        if (r < runs) scales[((size_t)p * D + j) * nb + b0 + r] = s_scale[e];
    }
}

}  // namespace

hipError_t launch_pack(const void* keys, int dtype, int P, int64_t n, int D, const float* rot,
                       uint64_t* planes, uint16_t* scales, hipStream_t st)
{
    const int64_t nb = (n + 63) / 64;
    dim3 grid((unsigned)((nb + kRun - 1) / kRun), (unsigned)P);
    if (dtype == 0) {
        if (rot) pack_kernel<0, true><<<grid, 256, 0, st>>>(keys, n, D, nb, rot, planes, scales);
        else pack_kernel<0, false><<<grid, 256, 0, st>>>(keys, n, D, nb, rot, planes, scales);
    } else {
        if (rot) pack_kernel<1, true><<<grid, 256, 0, st>>>(keys, n, D, nb, rot, planes, scales);
        else pack_kernel<1, false><<<grid, 256, 0, st>>>(keys, n, D, nb, rot, planes, scales);
    }
    return hipGetLastError();
}

}  // namespace fathom

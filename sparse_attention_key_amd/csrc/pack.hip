// Quantise keys into the channel-major bit-plane index (yeyulingfeng.com
// write-up of Fathom, section "方法一": per-channel uniform symmetric 4-bit
// code, one fp16 scale per 64-token block, bit p of the block's 64 codes in
// one 64-bit plane word, planes laid out along the sequence per channel).
//
// One workgroup (4 wavefronts) packs up to 8 consecutive blocks of one pair,
// one block at a time: the block's 64 keys are read with coalesced 16-byte
// loads into LDS, then the wavefronts share out the channels -- lane i =
// token i, so the block max of a channel is a wavefront max-reduction and
// each plane word is one ballot.  Words are collected in LDS as
// [channel][plane][blocks] and written out as whole row segments, so the
// scattered per-block words never hit HBM one by one.  Without rotation
// the channels of a block are split over CG = 4 workgroups, each staging
// and quantising its quarter, so that more blocks are in flight.
#include "common.h"

namespace fathom {
namespace {

constexpr int kRun = 8;  // blocks per workgroup
constexpr int kKeyStride = kMaxD + 1;  // LDS row of one token's keys (padded)

// Exact floor(x / delta) + 8, clamped to the 4-bit range.  delta = scale/8
// has at most 11 significant bits and |x / delta| stays below ~9 inside a
// block, so f * delta is exact and two comparisons repair the rounding of
// x * inv, for any inv within a few ulp of 1/delta (the hardware
// reciprocal's error, ~1 ulp, moves x * inv by far less than one).
__device__ __forceinline__ uint32_t quant_code(float x, float delta, float inv)
{
    if (!(delta > 0.0f)) return 8u;
    float f = floorf(x * inv);
    if (f * delta > x) f -= 1.0f;
    else if ((f + 1.0f) * delta <= x) f += 1.0f;
    f = fminf(fmaxf(f + 8.0f, 0.0f), 15.0f);
    return (uint32_t)f;
}

// Copies channels [c0, c0 + DG) of the keys of tokens [t0, t0 + 64) (those
// below m) of pair p into s_keys[token][channel - c0] (rows of `ks` floats),
// with 16-byte loads along each row (c0 and DG multiples of 8).
template <int DTYPE>
__device__ __forceinline__ void stage_keys(const void* keys, int64_t m, int D, int c0, int DG, int p,
                                           int64_t t0, float* s_keys, int ks)
{
    constexpr int per = DTYPE == 0 ? 4 : 8;  // elements per 16-byte load
    const int vecs = DG / per;
    for (int e = threadIdx.x; e < 64 * vecs; e += blockDim.x) {
        const int i = e / vecs, c = (e - i * vecs) * per;
        const int64_t tok = t0 + i;
        float v[8];
        if (tok < m) {
            const size_t off = ((size_t)p * m + (size_t)tok) * D + c0 + c;
            if (DTYPE == 0) {
                const float4 f = *reinterpret_cast<const float4*>((const float*)keys + off);
                v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
            } else {
                const uint4 u = *reinterpret_cast<const uint4*>((const uint16_t*)keys + off);
                const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {  // bfloat16 widens exactly
                    v[2 * k] = __uint_as_float(w[k] << 16);
                    v[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
                }
            }
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) v[k] = 0.0f;
        }
#pragma unroll
        for (int k = 0; k < per; ++k) s_keys[i * ks + c + k] = v[k];
    }
}

// Scalar fallback for D not a multiple of 8 (one element per load).
template <int DTYPE>
__device__ __forceinline__ void stage_keys_scalar(const void* keys, int64_t m, int D, int p,
                                                  int64_t t0, float* s_keys)
{
    for (int e = threadIdx.x; e < 64 * D; e += blockDim.x) {
        const int i = e / D, c = e - i * D;
        const int64_t tok = t0 + i;
        float v = 0.0f;
        if (tok < m) {
            const size_t off = ((size_t)p * m + (size_t)tok) * D + c;
            v = DTYPE == 0 ? ((const float*)keys)[off]
                           : __uint_as_float((uint32_t)((const uint16_t*)keys)[off] << 16);
        }
        s_keys[i * kKeyStride + c] = v;
    }
}

// Blocks [b0, b0 + nbk) of every pair, from the m keys [P][m][D] that start
// at token 64 * b0; the index rows hold ldb blocks.  With CG > 1 the
// workgroup packs channels [z DG, z DG + DG) only (z = blockIdx.z, DG =
// D / CG, a multiple of 8; no rotation, which needs whole rows).
template <int DTYPE, bool ROT, int CG>
__global__ __launch_bounds__(256) void pack_kernel(const void* __restrict__ keys, int64_t m,
                                                   int D, int64_t bfirst, int64_t nbk, int64_t ldb,
                                                   const float* __restrict__ rot,
                                                   uint64_t* __restrict__ planes,
                                                   uint16_t* __restrict__ scales)
{
    constexpr int kDG = kMaxD / CG;                        // channels per workgroup (at most)
    constexpr int kKS = CG == 1 ? kKeyStride : kDG + 1;    // LDS row of one token's keys (padded)
    __shared__ uint64_t s_words[kDG * 4 * kRun];           // 32 KB / CG
    __shared__ uint16_t s_scale[kDG * kRun];
    __shared__ float s_keys[64 * kKS];                     // 33 KB / CG

    const int p = blockIdx.y;
    const int64_t b0 = (int64_t)blockIdx.x * kRun;  // relative to bfirst
    const int wave = threadIdx.x / kWave, lane = lane_id();
    const float* U = ROT ? rot + (size_t)p * D * D : nullptr;
    const int runs = (int)((nbk - b0) < kRun ? (nbk - b0) : kRun);
    const int DG = CG == 1 ? D : D / CG, c0 = CG == 1 ? 0 : (int)blockIdx.z * DG;

    for (int r = 0; r < runs; ++r) {
        const int64_t tok = (b0 + r) * 64 + lane;  // position among the m keys
        const bool valid = tok < m;
        if (CG > 1 || D % 8 == 0) stage_keys<DTYPE>(keys, m, D, c0, DG, p, (b0 + r) * 64, s_keys, kKS);
        else stage_keys_scalar<DTYPE>(keys, m, D, p, (b0 + r) * 64, s_keys);
        __syncthreads();
        const float* kr = s_keys + lane * kKS;
        for (int jl = wave; jl < DG; jl += 4) {
            float x;
            if (ROT) {
                float acc = 0.0f;
                for (int d = 0; d < D; ++d) acc = __builtin_fmaf(U[(size_t)d * D + jl], kr[d], acc);
                x = acc;
            } else {
                x = kr[jl];
            }
            const float mx = wave_max_f32(valid ? fabsf(x) : 0.0f);
            const uint32_t sb = f32_to_f16_rne_sat(mx);
            const float delta = f16_bits_to_f32(sb) * 0.125f;
            const float inv = __builtin_amdgcn_rcpf(delta);
            const uint32_t c = valid ? quant_code(x, delta, inv) : 8u;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const uint64_t word = __ballot((c >> (3 - s)) & 1u);
                if (lane == 0) s_words[(jl * 4 + s) * kRun + r] = word;
            }
            if (lane == 0) s_scale[jl * kRun + r] = (uint16_t)sb;
        }
        __syncthreads();  // s_keys is refilled for the next block
    }

    for (int e = threadIdx.x; e < DG * 4 * kRun; e += blockDim.x) {
        const int r = e % kRun, js = e / kRun;
        if (r < runs) planes[((size_t)p * D * 4 + (size_t)c0 * 4 + js) * ldb + bfirst + b0 + r] = s_words[e];
    }
    for (int e = threadIdx.x; e < DG * kRun; e += blockDim.x) {
        const int r = e % kRun, j = e / kRun;
        if (r < runs) scales[((size_t)p * D + c0 + j) * ldb + bfirst + b0 + r] = s_scale[e];
    }
}

}  // namespace

hipError_t launch_pack(const void* keys, int dtype, int P, int64_t tok0, int64_t m, int D,
                       const float* rot, uint64_t* planes, uint16_t* scales, int64_t ldb,
                       hipStream_t st)
{
    const int64_t bfirst = tok0 / 64, nbk = (m + 63) / 64;
    const int64_t gx = (nbk + kRun - 1) / kRun;
    // the channels of a block split over four workgroups (each stages and
    // quantises a quarter of them): more, smaller workgroups keep more blocks
    // in flight (8 pairs x 1M bf16 keys: 5.9 ms unsplit, 2.3 ms split; eight
    // ways 2.4 ms; an append of one block per pair: 29.6 us unsplit, 13 us)
    const bool split = !rot && D % 32 == 0;
    const dim3 grid((unsigned)gx, (unsigned)P, split ? 4u : 1u);
#define FATHOM_PACK(DT, R, CG) pack_kernel<DT, R, CG><<<grid, 256, 0, st>>>(keys, m, D, bfirst, nbk, ldb, rot, planes, scales)
    if (dtype == 0) {
        if (rot) FATHOM_PACK(0, true, 1);
        else if (split) FATHOM_PACK(0, false, 4);
        else FATHOM_PACK(0, false, 1);
    } else {
        if (rot) FATHOM_PACK(1, true, 1);
        else if (split) FATHOM_PACK(1, false, 4);
        else FATHOM_PACK(1, false, 1);
    }
#undef FATHOM_PACK
    return hipGetLastError();
}

}  // namespace fathom

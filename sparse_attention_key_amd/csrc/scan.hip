// Approximate scores of every key from the bit-plane index, on the matrix
// cores (yeyulingfeng.com write-up of Fathom: section "方法一" -- a t-plane
// prefix is the t-bit mid-rise quantiser; section "方法二" -- only the first
// t_j planes of each active channel are read, and the plan is shared by the
// G heads of a group so the index is read once for all of them).
//
// Score contract (fixed point: the sum is exact, only the result is rounded).
// Per pair and head h, sigma_h = 31 - floor(log2 max_j |q_hj|) over the read
// channels; per 64-token block b, E_b = floor(log2) of the largest scale of
// the read channels (0 when it is 0).  Each read channel gets the integer
// coefficient A_hjb = trunc(fl32(fl32(q_hj 2^sigma_h) * scale_jb) *
// 2^-(E_b+3)), |A| <= 2^30.  With c' = c_t 2^(4-t) (the prefix code with
// zeros below it) the prefix key is (2 c' + 2^(4-t) - 16) scale / 16, so
//     S = sum_j A_hjb (2 c'_j + 2^(4-t_j) - 16)
// is an exact integer and the score is fl32(S 2^(E_b - 1 - sigma_h)).
//
// How the sum reaches the matrix cores.  A coefficient is split into four
// signed bytes (balanced base-256 digits: the bytes of (A + 0x808080) ^
// 0x808080), and v_mfma_i32_16x16x{32,64}_i8 multiplies a 16 x K tile of
// digits (rows: 4 heads x 4 digits) by a K x 16 tile of codes (columns: 16
// tokens of one block) with exact int32 sums; the four digit rows of a head
// recombine into S.  K runs over "slots": the active channels sorted by depth
// (deepest first), padded with zero coefficients to S_slots = 32, 64 or 128.
// The constant sum_j A_hjb (2^(4-t_j) - 16) is one more product per block,
// of the same digit tile with a column of those constants.
//
// Codes.  A wavefront takes 4/C blocks at a time (C = S_slots / 32).  A lane
// extracts the codes of one (slot, half block) -- 32 tokens -- from the
// slot's plane words with SWAR shifts: group g (tokens g, g+8, g+16, g+24,
// one per byte) lands with its sign plane on bit m_g of the byte (m = 3 for
// groups 3 and 7, 4 for 0 and 4, 5 for 1 and 5, 6 for 2 and 6), so one
// shift per plane and direction serves every group and each byte holds
// c' 2^(m_g - 3).  The 32 code bytes go to LDS as four 8-byte chunks of
// equal weight; ds_read_b64_tr_b8 then transposes 16 such rows (8 slots x 2
// halves) into the operand layout (each lane: one token, 8 slots), so the
// codes never need an in-register transpose.  The per-chunk weight 2^rho is
// undone when the sum is recombined.
//
// Output modes: STORE writes every score; FILTER keeps the scores at or
// above the per-head threshold as 64-bit (key, ~index) candidates (an exact
// integer bound on the top digits screens the tokens, survivors get their
// exact score); LANEMAX writes, per block and head, the maxima of four
// groups of 16 tokens (the input of the top-k threshold).
#include "common.h"

namespace fathom {
namespace {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned short us2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kWaveBlocks = 64;                    // logical blocks per wavefront
constexpr int kGroupBlocks = kWaves * kWaveBlocks;  // per workgroup
constexpr int kRun = 32;                           // sampled blocks come in runs of 32
constexpr int kSlotsMax = 128;
constexpr int kRec = 32;                           // LDS bytes per (slot, half block) code record
constexpr int kCodeBytes = 8 * 32 * kRec;          // 2 (4/C) half blocks x 32 C slots, every C
constexpr int kCoefBytes = 4 * 32 * 16;            // (4/C) blocks x 32 C slots x 2 head pairs x 8 B
constexpr int kStage = 32;                         // staged survivors per head and wavefront

enum { kStore = 0, kFilter = 1, kLaneMax = 2 };

typedef __attribute__((address_space(3))) v2i lds_v2i;

__device__ __forceinline__ v2i tr8(const unsigned char* base, uint32_t off)
{
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(base + off));
}

__device__ __forceinline__ long as_long(v2i v) { return __builtin_bit_cast(long, v); }

// sum over the K slots of digit rows x code columns; C = 1: K = 32, 2: K = 64,
// 4: two K = 64 products
__device__ __forceinline__ v4i mfma_k(const v2i (&a)[4], const v2i (&b)[4], int C)
{
    const v4i z = {0, 0, 0, 0};
    if (C == 1) return __builtin_amdgcn_mfma_i32_16x16x32_i8(as_long(a[0]), as_long(b[0]), z, 0, 0, 0);
    const v4i a0 = {a[0].x, a[0].y, a[1].x, a[1].y}, b0 = {b[0].x, b[0].y, b[1].x, b[1].y};
    v4i r = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b0, z, 0, 0, 0);
    if (C == 4) {
        const v4i a1 = {a[2].x, a[2].y, a[3].x, a[3].y}, b1 = {b[2].x, b[2].y, b[3].x, b[3].y};
        r = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b1, r, 0, 0, 0);
    }
    return r;
}

// The four digit sums of one (head, token) recombined: 2^rho (S - K) / 2
// split as hi * 2^16 + lo, both exact in int32.
__device__ __forceinline__ int64_t recombine(v4i o)
{
    const int lo = o.x + o.y * 256, hi = o.z + o.w * 256;
    return (int64_t)hi * 65536 + lo;
}

// exact score of a token from its digit sums (weight 2^rho) and the block
// constant (weight 1): S = 2 X + K with o = 2^rho X
__device__ __forceinline__ float exact_score(v4i o, int64_t K, int rho, int zeta)
{
    const int64_t x = recombine(o);
    const int64_t S = (rho == 0 ? x * 2 : (x >> (rho - 1))) + K;
    return (float)__builtin_ldexp((double)S, zeta);
}

// sign-plane position of byte group g (see the file comment)
__host__ __device__ constexpr int group_msb(int g) { return g == 7 ? 3 : g >= 3 ? g : g + 4; }

// Codes of one (slot, half block) from its plane words (absent planes are
// zero words), straight into the four 8-byte chunks of its LDS record:
// chunk rho holds groups (3, 7), (0, 4), (1, 5), (2, 6) for rho = 0..3, and
// byte k of group g is c' 2^(m_g - 3) of token g + 8k.  Plane 0 is always
// read (a step with no slot to read has zero words).
__device__ __forceinline__ void extract(const uint32_t (&w)[4], int tmax, v2i (&ch)[4])
{
    constexpr uint32_t M = 0x01010101u;
    {
        const uint32_t r = w[0], l = w[0] << 4, r4 = w[0] >> 4;
        ch[0].x = (int)(r & (M << group_msb(3)));
        ch[0].y = (int)(r4 & (M << group_msb(7)));
        ch[1].x = (int)(l & (M << group_msb(0)));
        ch[1].y = (int)(r & (M << group_msb(4)));
        ch[2].x = (int)(l & (M << group_msb(1)));
        ch[2].y = (int)(r & (M << group_msb(5)));
        ch[3].x = (int)(l & (M << group_msb(2)));
        ch[3].y = (int)(r & (M << group_msb(6)));
    }
#pragma unroll
    for (int s = 1; s < 4; ++s) {
        if (s < tmax) {  // wavefront-uniform
            const uint32_t r = w[s] >> s, l = w[s] << (4 - s), r4 = w[s] >> (4 + s);
            ch[0].x |= (int)(r & (M << (group_msb(3) - s)));
            ch[0].y |= (int)(r4 & (M << (group_msb(7) - s)));
            ch[1].x |= (int)(l & (M << (group_msb(0) - s)));
            ch[1].y |= (int)(r & (M << (group_msb(4) - s)));
            ch[2].x |= (int)(l & (M << (group_msb(1) - s)));
            ch[2].y |= (int)(r & (M << (group_msb(5) - s)));
            ch[3].x |= (int)(l & (M << (group_msb(2) - s)));
            ch[3].y |= (int)(r & (M << (group_msb(6) - s)));
        }
    }
}

// LDS layout of the codes.  Record (block b, half hs, slot e) -- 32 bytes,
// four 8-byte chunks rho of weight 2^rho -- sits at ((2b + hs) S + e) * 32,
// and chunk rho at position (rho + skew) & 3 within it, skew = e + e/8 +
// 2 hs + b: the 16 rows of a transposing read (8 slots x 2 halves) and the
// 32 records written by half a wavefront then fall on distinct banks.
__device__ __forceinline__ int rec_skew(int e, int hs, int b) { return (e + (e >> 3) + 2 * hs + b) & 3; }

template <int GR>
struct PairTables {
    uint32_t slot[kSlotsMax];                               // channel | depth << 8, deepest first
    __attribute__((aligned(8))) signed char d[kSlotsMax];   // 2^(4-t) - 16 per slot (0 past A)
    int sig[4 * GR];
    uint32_t qmax[4 * GR];
    uint32_t cnt[5];
};

// wavefront max of a non-negative value, through DPP row operations
__device__ __forceinline__ int wave_max_dpp(int v)
{
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false));  // row_half_mirror
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false));  // row_mirror
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false));  // row_bcast15
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false));  // row_bcast31
    return __builtin_amdgcn_readlane(v, 63);
}

template <int GR, int MODE, int C>
__device__ __forceinline__ void scan_body(const ScanArgs& a, const int p, const int G, const int A,
                                          const PairTables<GR>& T, unsigned char* code,
                                          unsigned char* coef, uint64_t* stage, uint32_t* wcnt)
{
    constexpr int S = 32 * C, NB = 4 / C;
    constexpr int NH = 4 * GR;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    const int kap = lane >> 4, j16 = lane & 15;  // lane group (slot block / head) and row
    // block indices fit 32 bits (the host checks the index size)
    const int nlb = (int)a.nlb, nbk = (int)a.nb, stride = (int)a.stride;
    const int lwave0 = ((int)blockIdx.x * kWaves + wave) * kWaveBlocks;  // first logical block
    if (lwave0 >= nlb) return;
    const int lend = min(lwave0 + kWaveBlocks, nlb);
    const int64_t ldb = a.ldb;

    // buffer descriptors of the pair's planes and scales
    const uint64_t* pplanes = a.planes + (size_t)p * a.D * 4 * ldb;
    const uint16_t* pscales = a.scales + (size_t)p * a.D * ldb;
    const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
        (void*)pplanes, (short)0, (int)((int64_t)a.D * 4 * ldb * 8), 0x00020000);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)pscales, (short)0, (int)((int64_t)a.D * ldb * 2), 0x00020000);
    constexpr uint32_t kOOB = 0x80000000u;  // past every record: the load returns 0
    const uint32_t ldb8 = (uint32_t)(ldb * 8);

    // ---- codes: at step u the wavefront extracts slots 8C u .. 8C u + 8C-1
    // of every half block; lane L takes slot 8C u + L % 8C, half (L / 8C) % 2
    // of block L / 16C
    const int tsl = lane % (8 * C), ths = (lane / (8 * C)) & 1, tbk = lane / (16 * C);
    uint32_t trow[4];  // plane-0 byte offset of the task's row (+ half), or out of range
    int tt[4], tmax[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int e = 8 * C * u + tsl;
        tt[u] = (int)(T.slot[e] >> 8);
        trow[u] = tt[u] ? (uint32_t)(T.slot[e] & 255u) * 4u * ldb8 + (uint32_t)ths * 4u : kOOB;
        tmax[u] = __builtin_amdgcn_readfirstlane((int)(T.slot[8 * C * u] >> 8));  // deepest at step u
    }
    // record write offsets: chunk rho of step u goes to wr[(rho + C u) & 3] + u * 8C * 32
    uint32_t wr[4];
    {
        const int sk = rec_skew(tsl, ths, tbk);
        const uint32_t base = (uint32_t)(((2 * tbk + ths) * S + tsl) * kRec);
#pragma unroll
        for (int m = 0; m < 4; ++m) wr[m] = base + (uint32_t)(((m + sk) & 3) * 8);
    }
    // transposing read offsets: read r of tile (b, rho) is rd[r][(rho + b) & 3] + 2 b S 32
    uint32_t rd[C][4];
#pragma unroll
    for (int r = 0; r < C; ++r) {
        const int e = 32 * r + 8 * kap + (j16 >> 1), hs = j16 & 1;
        const int sk = rec_skew(e, hs, 0);
        const uint32_t base = (uint32_t)((hs * S + e) * kRec);
#pragma unroll
        for (int m = 0; m < 4; ++m) rd[r][m] = base + (uint32_t)(((m + sk) & 3) * 8);
    }
    // ---- digit rows: the 16C lanes of block L / 16C compute its (slot,
    // head pair) rows pi = L % 16C + 16C k, k = 0..3 (slot pi / 2, pair L & 1)
    constexpr int LPB = 16 * C;
    const int rb = lane / LPB, rl = lane % LPB, rhp = lane & 1;
    uint32_t srow[4];  // scale row byte offset of slot k (out of range past A)
    float qt[4][GR][2];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int e = (rl >> 1) + 8 * C * k;
        const int j = (int)(T.slot[e] & 255u);
        srow[k] = e < A ? (uint32_t)j * (uint32_t)(ldb * 2) : kOOB;
#pragma unroll
        for (int gr = 0; gr < GR; ++gr)
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const int h = 4 * gr + 2 * rhp + x;
                qt[k][gr][x] = (e < A && h < G)
                    ? __builtin_ldexpf(a.q_used[((size_t)p * G + h) * a.D + j], T.sig[h]) : 0.0f;
            }
    }
    // constants column of read r: slots 32 r + 8 kap + 0..7
    v2i dcol[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) dcol[r] = r < C ? *(const v2i*)(T.d + 32 * r + 8 * kap) : (v2i){0, 0};
    // screen margins (hi units, 2^16): the two lower digit sums of a tile of
    // weight 2^rho are bounded by 15 2^rho (128 * 256 + 128) A, those of the
    // block constant by 15 (128 * 256 + 128) A
    const float lob = 7.53f * (float)A + 1.0f;
    // per-lane heads kap + 4 gr
    float thr[GR], pth[GR];
    int sig[GR];
#pragma unroll
    for (int gr = 0; gr < GR; ++gr) {
        const int h = kap + 4 * gr;
        sig[gr] = T.sig[h];
        thr[gr] = pth[gr] = INFINITY;
        if (MODE == kFilter && h < G) {
            const uint32_t tk = a.tau[(size_t)p * G + h];
            const float th = tk <= 0x007FFFFFu ? -INFINITY : key_score(tk);
            thr[gr] = th;
            // next float below the threshold: a score >= th has S 2^zeta above it
            pth[gr] = th == -INFINITY ? -INFINITY
                    : th > 0.0f  ? __uint_as_float(__float_as_uint(th) - 1u)
                    : th == 0.0f ? -1.40129846e-45f
                                 : __uint_as_float(__float_as_uint(th) + 1u);
        }
    }
    if (MODE == kFilter && lane < NH) wcnt[lane] = 0u;
    // token offset (within its block) of this lane's column in chunk rho
    int toff[4];
#pragma unroll
    for (int rho = 0; rho < 4; ++rho) {
        const int x = j16 & 7;
        const int g = x < 4 ? (rho == 0 ? 3 : rho - 1) : (rho == 0 ? 7 : rho + 3);
        toff[rho] = 32 * (j16 >> 3) + g + 8 * (x & 3);
    }

    // physical block of a logical one: runs of kRun, one run in every stride.
    // The NB blocks of an iteration lie in one run, so they are consecutive;
    // blocks past the index read as zeros (the buffer bound) and are masked.
    auto phys = [&](int lb) { return (lb / kRun) * kRun * stride + (lb % kRun); };
    auto issue = [&](int lb0, uint32_t (&w)[4][4], uint32_t (&scl)[4]) {
        const uint32_t pb0 = (uint32_t)phys(lb0);
        const uint32_t pb8 = (pb0 + (uint32_t)tbk) * 8u;
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                w[u][s] = 0;
                if (s < tmax[u]) {
                    const uint32_t off = s < tt[u] ? trow[u] + (uint32_t)s * ldb8 + pb8 : kOOB;
                    w[u][s] = __builtin_amdgcn_raw_buffer_load_b32(rp, off, 0, 0);
                }
            }
#pragma unroll
        for (int k = 0; k < 4; ++k)
            scl[k] = __builtin_amdgcn_raw_buffer_load_b16(rs, srow[k] + (pb0 + (uint32_t)rb) * 2u, 0, 0) & 0xFFFFu;
    };

    uint32_t wn[4][4], scn[4];
    issue(lwave0, wn, scn);
    for (int lb0 = lwave0; lb0 < lend; lb0 += NB) {
        uint32_t w[4][4], scl[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int s = 0; s < 4; ++s) w[u][s] = wn[u][s];
#pragma unroll
        for (int k = 0; k < 4; ++k) scl[k] = scn[k];
        if (lb0 + NB < lend) issue(lb0 + NB, wn, scn);  // next iteration's loads in flight

        int pbk[NB], nval[NB];  // physical block, and its valid tokens (0 for dead blocks)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int lb = lb0 + b;
            pbk[b] = phys(lb);
            const int64_t left = a.n - (int64_t)pbk[b] * 64;
            nval[b] = (lb < nlb && pbk[b] < nbk) ? (int)(left < 64 ? left : 64) : 0;
        }

        // ---- codes to LDS (a step with no slot to read is skipped: its
        // records meet zero coefficients)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (tmax[u] == 0) continue;
            v2i ch[4];
            extract(w[u], tmax[u], ch);
#pragma unroll
            for (int rho = 0; rho < 4; ++rho)
                *(v2i*)(code + wr[(rho + C * u) & 3] + u * 8 * C * kRec) = ch[rho];
        }

        // ---- block exponents: largest exponent field of the read scales (>= 1),
        // reduced over the lanes of the block's row group
        int ef = 1;
#pragma unroll
        for (int k = 0; k < 4; ++k) ef = max(ef, (int)((scl[k] >> 10) & 31u));
        ef = max(ef, __builtin_amdgcn_update_dpp(0, ef, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
        ef = max(ef, __builtin_amdgcn_update_dpp(0, ef, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
        ef = max(ef, __builtin_amdgcn_update_dpp(0, ef, 0x141, 0xF, 0xF, false));  // row_half_mirror
        ef = max(ef, __builtin_amdgcn_update_dpp(0, ef, 0x140, 0xF, 0xF, false));  // row_mirror
        if (C >= 2) ef = max(ef, __shfl_xor(ef, 16, kWave));
        if (C >= 4) ef = max(ef, __shfl_xor(ef, 32, kWave));
        int Eb[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) Eb[b] = __builtin_amdgcn_readlane(ef, b * LPB) - 15;
        const int Erow = ef - 15;  // the lane's own block

        // ---- digit rows to LDS
        {
            const float pw = __uint_as_float((uint32_t)(127 - Erow - 3) << 23);  // 2^-(E+3)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int e = (rl >> 1) + 8 * C * k;
                const float sc = (float)__builtin_bit_cast(_Float16, (uint16_t)scl[k]);
#pragma unroll
                for (int gr = 0; gr < GR; ++gr) {
                    uint32_t dig[2];
#pragma unroll
                    for (int x = 0; x < 2; ++x) {
                        // trunc(fl32(q 2^sigma * scale) 2^-(E+3)); q 2^sigma 2^-(E+3) is exact
                        const int Ai = (int)((qt[k][gr][x] * pw) * sc);
                        dig[x] = ((uint32_t)Ai + 0x00808080u) ^ 0x00808080u;
                    }
                    *(v2i*)(coef + gr * kCoefBytes + rb * (S * 16) + (e * 2 + rhp) * 8) =
                        (v2i){(int)dig[0], (int)dig[1]};
                }
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // ---- products per block
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int lb = lb0 + b;
            v2i ac[GR][4];
#pragma unroll
            for (int gr = 0; gr < GR; ++gr)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    ac[gr][r] = r < C ? tr8(coef + gr * kCoefBytes,
                                            (uint32_t)(b * (S * 16) + ((32 * r + 8 * kap + (j16 >> 1)) * 2 + (j16 & 1)) * 8))
                                      : (v2i){0, 0};
            v4i kk[GR];
            float hv[GR][4];
            int64_t smax[GR];
#pragma unroll
            for (int gr = 0; gr < GR; ++gr) {
                kk[gr] = mfma_k(ac[gr], dcol, C);
                smax[gr] = INT64_MIN;
            }
            v2i bc[4][4];
#pragma unroll
            for (int rho = 0; rho < 4; ++rho)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    bc[rho][r] = r < C ? tr8(code, rd[r][(rho + b) & 3] + (uint32_t)(2 * b * S * kRec))
                                       : (v2i){0, 0};
            v4i o[4][GR];
#pragma unroll
            for (int rho = 0; rho < 4; ++rho)
#pragma unroll
                for (int gr = 0; gr < GR; ++gr) o[rho][gr] = mfma_k(ac[gr], bc[rho], C);
            if (MODE == kFilter) {
                // Screen, per tile rho: a token whose exact S passes has
                // fl(hi) >= hv = 2^(rho-1) (P - K) / 2^16 - bound(lo), with
                // P = pred(th) 2^-zeta; hv is a float lower bound of that.
#pragma unroll
                for (int gr = 0; gr < GR; ++gr) {
                    const float phi = __builtin_ldexpf(pth[gr], sig[gr] - 15 - Eb[b]);
                    const float z = phi - (float)(kk[gr].z + kk[gr].w * 256);
                    const float zf = z - lob - 4.0f - fabsf(z) * (1.0f / 262144.0f);
#pragma unroll
                    for (int rho = 0; rho < 4; ++rho)
                        hv[gr][rho] = __builtin_fmaf(zf, rho == 0 ? 0.5f : (float)(1 << (rho - 1)),
                                                     -(lob * (float)(1 << rho) + 2.0f));
                }
                const bool fullb = nval[b] == 64;
                auto passes = [&](int rho, int gr) {
                    const int hi = o[rho][gr].z + o[rho][gr].w * 256;
                    return (float)hi >= hv[gr][rho] && (fullb || toff[rho] < nval[b]) && kap + 4 * gr < G;
                };
                bool any = false;
#pragma unroll
                for (int rho = 0; rho < 4; ++rho)
#pragma unroll
                    for (int gr = 0; gr < GR; ++gr) any |= passes(rho, gr);
                if (any) {  // rare: exact scores of the survivors
#pragma unroll
                    for (int rho = 0; rho < 4; ++rho)
#pragma unroll
                        for (int gr = 0; gr < GR; ++gr) {
                            if (!passes(rho, gr)) continue;
                            const int h = kap + 4 * gr;
                            const float sc = exact_score(o[rho][gr], recombine(kk[gr]), rho, Eb[b] - 1 - sig[gr]);
                            if (sc >= thr[gr]) {
                                const uint32_t tok = (uint32_t)pbk[b] * 64u + (uint32_t)toff[rho];
                                const uint64_t cv = composite(score_key(sc), tok);
                                const uint32_t pos = atomicAdd(&wcnt[h], 1u);
                                if (pos < (uint32_t)kStage) {
                                    stage[h * kStage + pos] = cv;
                                } else {
                                    const uint32_t slot = atomicAdd(&a.counts[(size_t)p * G + h], 1u);
                                    if ((int64_t)slot < a.cap) a.cand[((size_t)p * G + h) * a.cap + slot] = cv;
                                }
                            }
                        }
                }
            } else {
#pragma unroll
                for (int rho = 0; rho < 4; ++rho) {
                    const bool tval = toff[rho] < nval[b];
#pragma unroll
                    for (int gr = 0; gr < GR; ++gr) {
                        const int h = kap + 4 * gr;
                        const int64_t Kc = recombine(kk[gr]);
                        if (MODE == kStore) {
                            const float sc = exact_score(o[rho][gr], Kc, rho, Eb[b] - 1 - sig[gr]);
                            if (h < G && lb < nlb)
                                a.out[((size_t)p * G + h) * (a.nlb * 64) + (int64_t)lb * 64 + toff[rho]] =
                                    tval ? sc : -INFINITY;
                        } else {
                            // the block's tokens share zeta: the largest S has the largest score
                            const int64_t x = recombine(o[rho][gr]);
                            const int64_t Sv = (rho == 0 ? x * 2 : (x >> (rho - 1))) + Kc;
                            if (tval && Sv > smax[gr]) smax[gr] = Sv;
                        }
                    }
                }
            }
            if (MODE == kLaneMax) {
                // maxima of 16 tokens: lanes 4q .. 4q+3 of a head
#pragma unroll
                for (int gr = 0; gr < GR; ++gr) {
                    float v = smax[gr] == INT64_MIN ? -INFINITY
                            : (float)__builtin_ldexp((double)smax[gr], Eb[b] - 1 - sig[gr]);
                    v = fmaxf(v, __shfl_xor(v, 1, kWave));
                    v = fmaxf(v, __shfl_xor(v, 2, kWave));
                    const int h = kap + 4 * gr;
                    if ((j16 & 3) == 0 && h < G && lb < nlb)
                        a.out[((size_t)p * G + h) * (a.nlb * 4) + (int64_t)lb * 4 + (j16 >> 2)] = v;
                }
            }
        }
        __builtin_amdgcn_wave_barrier();  // the next iteration rewrites this wavefront's LDS
    }
    if (MODE == kFilter) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        uint32_t nh = 0, base = 0;
        if (lane < NH && lane < G) {
            nh = min(wcnt[lane], (uint32_t)kStage);
            if (nh) base = atomicAdd(&a.counts[(size_t)p * G + lane], nh);
        }
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            const uint32_t n_h = (uint32_t)__builtin_amdgcn_readlane((int)nh, h);
            const uint32_t b_h = (uint32_t)__builtin_amdgcn_readlane((int)base, h);
            if ((uint32_t)lane < n_h && (int64_t)(b_h + lane) < a.cap)
                a.cand[((size_t)p * G + h) * a.cap + b_h + lane] = stage[h * kStage + lane];
        }
    }
}

template <int GR, int MODE>
__device__ __forceinline__ void scan_pair(const ScanArgs& a, const int p, const int G)
{
    constexpr int NH = 4 * GR;
    __shared__ PairTables<GR> T;
    __shared__ __attribute__((aligned(16))) unsigned char s_code[kWaves][kCodeBytes];
    __shared__ __attribute__((aligned(16))) unsigned char s_coef[kWaves][GR * kCoefBytes];
    __shared__ uint64_t s_stage[kWaves][NH * kStage];
    __shared__ uint32_t s_wcnt[kWaves][NH];

    const int lane = lane_id(), wave = threadIdx.x / kWave;
    const int A = a.n_active[p];

    // ---- pair tables: slots sorted by depth (counting sort), scaled queries
    if (threadIdx.x < 5) T.cnt[threadIdx.x] = 0u;
    if (threadIdx.x < NH) T.qmax[threadIdx.x] = 0u;
    __syncthreads();
    for (int e = threadIdx.x; e < A; e += kThreads) {
        const int j = a.active[(size_t)p * a.D + e];
        atomicAdd(&T.cnt[a.depth[(size_t)p * a.D + j]], 1u);
        for (int h = 0; h < G && h < NH; ++h)  // |q| bits order like |q| values
            atomicMax(&T.qmax[h], __float_as_uint(fabsf(a.q_used[((size_t)p * G + h) * a.D + j])));
    }
    __syncthreads();
    if (threadIdx.x == 0) {  // start of each depth class, deepest first
        uint32_t o = 0;
        for (int t = 4; t >= 1; --t) {
            const uint32_t c = T.cnt[t];
            T.cnt[t] = o;
            o += c;
        }
    }
    if (threadIdx.x < NH) {
        // sigma = 31 - floor(log2 max |q|), from the exponent field (subnormals lifted by 2^64)
        const float qm = __uint_as_float(T.qmax[threadIdx.x]);
        int sg = 0;
        if (qm > 0.0f) {
            const bool sub = qm < 1.17549435e-38f;
            const float qq = sub ? qm * 18446744073709551616.0f : qm;
            sg = 31 - ((int)((__float_as_uint(qq) >> 23) & 255u) - 127 - (sub ? 64 : 0));
        }
        T.sig[threadIdx.x] = sg;
    }
    __syncthreads();
    if (wave == 0) {  // slots of a depth class in ascending channel order
        for (int e0 = 0; e0 < A; e0 += kWave) {
            const int e = e0 + lane;
            int j = 0, t = 0;
            if (e < A) {
                j = a.active[(size_t)p * a.D + e];
                t = a.depth[(size_t)p * a.D + j];
            }
            for (int tt = 4; tt >= 1; --tt) {
                const uint64_t m = __ballot(e < A && t == tt);
                if (e < A && t == tt)
                    T.slot[T.cnt[tt] + __popcll(m & lanes_below(lane))] = (uint32_t)j | ((uint32_t)t << 8);
                __builtin_amdgcn_wave_barrier();
                if (lane == 0) T.cnt[tt] += (uint32_t)__popcll(m);
                __builtin_amdgcn_wave_barrier();
            }
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < kSlotsMax; e += kThreads) {
        int t = 0, j = 0;
        if (e < A) {
            j = (int)(T.slot[e] & 255u);
            t = (int)(T.slot[e] >> 8);
        } else {
            T.slot[e] = 0u;
        }
        (void)j;
        T.d[e] = (signed char)(e < A ? (1 << (4 - t)) - 16 : 0);
    }
    __syncthreads();

    unsigned char* code = s_code[wave];
    unsigned char* coef = s_coef[wave];
    uint64_t* stage = s_stage[wave];
    uint32_t* wcnt = s_wcnt[wave];
    if (A <= 32) scan_body<GR, MODE, 1>(a, p, G, A, T, code, coef, stage, wcnt);
    else if (A <= 64) scan_body<GR, MODE, 2>(a, p, G, A, T, code, coef, stage, wcnt);
    else scan_body<GR, MODE, 4>(a, p, G, A, T, code, coef, stage, wcnt);
}

// blockIdx.y is the pair; with a pair list (score mode only), the rows of
// the grid take the listed pairs in turn instead.
template <int GR, int MODE>
__global__ __launch_bounds__(kThreads) void scan_kernel(ScanArgs a, int G)
{
    if (MODE == kStore && a.list) {
        const uint32_t nlist = a.list[0];
        for (uint32_t r = blockIdx.y; r < nlist; r += gridDim.y) {
            scan_pair<GR, MODE>(a, (int)a.list[1 + r], G);
            __syncthreads();  // the pair's LDS tables are rewritten by the next one
        }
        return;
    }
    scan_pair<GR, MODE>(a, (int)blockIdx.y, G);
}

template <int MODE>
hipError_t launch_mode(const ScanArgs& a, int P, int G, hipStream_t st)
{
    const int rows = a.list ? (P < kListRows ? P : kListRows) : P;
    dim3 grid((unsigned)((a.nlb + kGroupBlocks - 1) / kGroupBlocks), (unsigned)rows);
    if (G <= 4) scan_kernel<1, MODE><<<grid, kThreads, 0, st>>>(a, G);
    else scan_kernel<2, MODE><<<grid, kThreads, 0, st>>>(a, G);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_scan_args(const ScanArgs& a, int P, int G, int mode, hipStream_t st)
{
    if (mode == kFilter) return launch_mode<kFilter>(a, P, G, st);
    if (mode == kLaneMax) return launch_mode<kLaneMax>(a, P, G, st);
    return launch_mode<kStore>(a, P, G, st);
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
    return launch_mode<kStore>(a, P, G, st);
}

}  // namespace fathom

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
#include "select.h"

namespace fathom {
namespace {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned short us2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kGroupBlocks = 1024;                 // logical blocks per workgroup (at most)
constexpr int kRunLog2 = 5;                        // sampled blocks come in runs of 32 (unless set)
constexpr int kSlotsMax = 128;
constexpr int kRec = 32;                           // LDS bytes per (slot, half block) code record
constexpr int kCodeBytes = 8 * 32 * kRec + 8 * 32;   // 2 (4/C) half blocks of 32 C slots and a spare record
// Bytes between the wavefronts' record areas.  A record write (16 lanes of
// 8 bytes per LDS pass: two slots x 8 block pairs, the pairs spread over the
// four areas) meets distinct banks when the areas are 32 bytes apart modulo
// the bank span (C = 1 and 2; two-way for C = 4): with no padding the four
// areas alias and the writes were four-way conflicted (47 conflict cycles
// per block at 1M tokens x 288 pairs).  Reads stay within one area, so the
// padding does not change them.
constexpr int kCodeStride = kCodeBytes + 32;
constexpr int kCoefBytes = 4 * 32 * 16;            // (4/C) blocks x 32 C slots x 2 head pairs x 8 B
constexpr int kStage = 128;                        // staged survivors per wavefront (16-byte records)

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
// four 8-byte chunks rho of weight 2^rho -- sits at (2b + hs) H + 32 e with
// H = 32 S + 32 (one spare record per half block), and chunk rho at
// position (rho + skew) & 3 within it, skew = e + 2 (e/4) + 2 (e/8) +
// 2 (b/2).  A 64-bit write goes 16 lanes at a time to 32 banks and a
// transposing read 32 lanes at a time to 64 banks (measured); with this
// layout the 16 records of a write pass (two slots x 8 half blocks, the
// lane order that keeps loads contiguous) and the 32 rows of a read pass
// all fall on distinct banks.  Step u of the writer holds slots 8 C u +
// tsl, whose skew is that of slot tsl plus 2 C u.
__device__ __forceinline__ int rec_skew(int e, int b) { return (e + 2 * (e >> 2) + 2 * (e >> 3) + 2 * (b >> 1)) & 3; }
template <int C> constexpr int kHalfBytes = 32 * 32 * C + 32;
template <int C> constexpr int kSkewStep = 2 * C;

template <int GR>
struct PairTables {
    uint32_t slot[kSlotsMax];                               // channel | depth << 8, deepest first
    __attribute__((aligned(8))) signed char d[kSlotsMax];   // 2^(4-t) - 16 per slot (0 past A)
    int sig[4 * GR];
    float thr[4 * GR];                                      // FILTER: the heads' thresholds
    uint32_t qmax[4 * GR];
    uint32_t cnt[5];
    float qv[4 * GR][kMaxD];                                // the heads' query values per channel
    short act[kMaxD];                                       // the active list (first A entries)
    unsigned char tch[kMaxD];                               // depth per channel
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

// Tile `tile` of pair p: logical blocks tile * gb .. tile * gb + gb - 1.
// STORE and LANEMAX write row `op` of the output (the pair itself, or a
// repair row).
template <int GR, int MODE, int C, bool STG>
__device__ __forceinline__ void scan_body(const ScanArgs& a, const int p, const int G, const int A,
                                          const int tile, const int op, const PairTables<GR>& T,
                                          unsigned char* code, unsigned char* coef, v4i* stage)
{
    constexpr int S = 32 * C, NB = 4 / C;
    constexpr int NH = 4 * GR;
    constexpr int IB = kWaves * NB;  // logical blocks the workgroup takes per iteration
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    const int kap = lane >> 4, j16 = lane & 15;  // lane group (slot block / head) and row
    // block indices fit 32 bits (the host caps n below 2^31 tokens), and the
    // plane and scale offsets below fit 31 bits (the host rejects a pair whose
    // plane rows span 2^31 bytes or more)
    const int nlb = (int)a.nlb, nbk = (int)a.nb, stride = (int)a.stride, skip = (int)a.skip;
    // Iteration i of wavefront w takes logical blocks lg0 + i IB + w NB + (0 .. NB-1):
    // at any time the four wavefronts of a workgroup read neighbouring blocks,
    // so each 128-byte line of a plane row is used by all of them at once.
    const int lg0 = tile * a.gb;
    const int lgend = min(lg0 + a.gb, nlb);
    if (lg0 + wave * NB >= lgend) return;
    const int64_t ldb = a.ldb;
    const uint32_t ldb8 = (uint32_t)(ldb * 8);

    // the pair's planes and scales; the descriptors are rebased on every
    // iteration's first physical block, so the range check stays exact
    const uint64_t* pplanes = a.planes + (size_t)p * a.D * 4 * ldb;
    const uint16_t* pscales = a.scales + (size_t)p * a.D * ldb;
    const uint32_t pbytes = (uint32_t)((int64_t)a.D * 4 * ldb * 8);
    const uint32_t sbytes = (uint32_t)((int64_t)a.D * ldb * 2);
    constexpr uint32_t kOOB = 0x80000000u;  // past every record: the load returns 0
    // (the record count is formed with a signed max: a saturating subtract
    // would be computed per lane and turn the descriptor into a per-lane value)
    auto records = [](uint32_t total, uint32_t off, bool live) {
        return __builtin_amdgcn_readfirstlane(live ? max((int)total - (int)off, 0) : 0);
    };
    // plane s of a row is read at the row's plane-0 offset (per lane) plus
    // s * ldb * 8 (the scalar offset); a lane whose block lies past the
    // index is pointed out of range (see `mask_dead`), so no read ever leaves
    // the pair's planes, whether or not the range check counts the scalar offset
    auto plane_rsrc = [&](int pb0, bool live) {
        const uint32_t off = (uint32_t)pb0 * 8u;
        return __builtin_amdgcn_make_buffer_rsrc((void*)((const unsigned char*)pplanes + off), (short)0,
                                                 records(pbytes, off, live), 0x00020000);
    };
    auto scale_rsrc = [&](int pb0, bool live) {
        const uint32_t off = (uint32_t)pb0 * 2u;
        return __builtin_amdgcn_make_buffer_rsrc((void*)((const unsigned char*)pscales + off), (short)0,
                                                 records(sbytes, off, live), 0x00020000);
    };

    // ---- codes: at step u the wavefront extracts slots 8C u .. 8C u + 8C-1
    // of every half block; lane L takes slot 8C u + L / 2NB, block (L / 2) %
    // NB, half L % 2, so neighbouring lanes read neighbouring words of a row
    const int tsl = lane / (2 * NB), tbk = (lane / 2) % NB, ths = lane & 1;
    uint32_t trow[4];  // byte offset of the task's plane-0 word from the iteration's first block
    int tt[4], tmax[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int e = 8 * C * u + tsl;
        tt[u] = (int)(T.slot[e] >> 8);
        trow[u] = tt[u] ? (uint32_t)(T.slot[e] & 255u) * 4u * ldb8 + (uint32_t)tbk * 8u + (uint32_t)ths * 4u : kOOB;
        tmax[u] = __builtin_amdgcn_readfirstlane((int)(T.slot[8 * C * u] >> 8));  // deepest at step u
    }
    // record write offsets: chunk rho of step u goes to wr[(rho + kSkewStep u) & 3] + u * 8C * 32
    uint32_t wr[4];
    {
        const int sk = rec_skew(tsl, tbk);
        const uint32_t base = (uint32_t)((2 * tbk + ths) * kHalfBytes<C> + tsl * kRec);
#pragma unroll
        for (int m = 0; m < 4; ++m) wr[m] = base + (uint32_t)(((m + sk) & 3) * 8);
    }
    // transposing read offsets: read r of tile (b, rho) is rd[r][(rho + 2 (b/2)) & 3] + 2 b H
    uint32_t rd[C][4];
#pragma unroll
    for (int r = 0; r < C; ++r) {
        const int e = 32 * r + 8 * kap + (j16 >> 1), hs = j16 & 1;
        const int sk = rec_skew(e, 0);
        const uint32_t base = (uint32_t)(hs * kHalfBytes<C> + e * kRec);
#pragma unroll
        for (int m = 0; m < 4; ++m) rd[r][m] = base + (uint32_t)(((m + sk) & 3) * 8);
    }
    // ---- digit rows: the 16C lanes of block L / 16C compute its (slot,
    // head pair) rows pi = L % 16C + 16C k, k = 0..3 (slot pi / 2, pair L & 1)
    constexpr int LPB = 16 * C;
    const int rb = lane / LPB, rl = lane % LPB, rhp = lane & 1;
    uint32_t srow[4];  // scale byte offset of slot k from the iteration's first block (out of range past A)
    float qt[4][GR][2];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int e = (rl >> 1) + 8 * C * k;
        const int j = (int)(T.slot[e] & 255u);
        srow[k] = e < A ? (uint32_t)j * (uint32_t)(ldb * 2) + (uint32_t)rb * 2u : kOOB;
#pragma unroll
        for (int gr = 0; gr < GR; ++gr)
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const int h = 4 * gr + 2 * rhp + x;
                qt[k][gr][x] = (e < A && h < G)
                    ? __builtin_ldexpf(T.qv[h][j], T.sig[h]) : 0.0f;
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
    // FILTER: screened tokens wait in this wavefront's stage as (exact sum,
    // token, head | exponent << 16) records; a flush turns them into scores,
    // keeps those at or above their head's threshold, and appends them to the
    // candidate lists with one fetch-and-add per head
    uint32_t scnt = 0;  // wavefront-uniform
    auto flush = [&]() {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        for (uint32_t r0 = 0; r0 < scnt; r0 += kWave) {
            const bool valid = r0 + (uint32_t)lane < scnt;
            v4i rec = valid ? stage[r0 + lane] : (v4i){0, 0, 0, 0};
            const int h = rec.w & 0xFF, zeta = rec.w >> 16;
            const int64_t S = (int64_t)(((uint64_t)(uint32_t)rec.y << 32) | (uint32_t)rec.x);
            const float sc = (float)__builtin_ldexp((double)S, zeta);
            const bool keep = valid && sc >= T.thr[h];
            const uint64_t cv = composite(score_key(sc), (uint32_t)rec.z);
            uint32_t nh = 0, mine = 0;
            uint64_t mh[NH];
#pragma unroll
            for (int hh = 0; hh < NH; ++hh) {
                mh[hh] = __builtin_amdgcn_ballot_w64(keep && h == hh);
                if (lane == hh) nh = (uint32_t)__popcll(mh[hh]);
                if (h == hh) mine = (uint32_t)__popcll(mh[hh] & lanes_below(lane));
            }
            uint32_t base = 0;
            if (lane < NH && lane < G && nh) base = atomicAdd(&a.counts[(size_t)p * G + lane], nh);
            const uint32_t bh = (uint32_t)__shfl((int)base, h, kWave);
            if (keep && (int64_t)(bh + mine) < a.cap) a.cand[((size_t)p * G + h) * a.cap + bh + mine] = cv;
        }
        scnt = 0;
    };
    // lanes of existing heads, per head group
    uint64_t hmask[GR];
#pragma unroll
    for (int gr = 0; gr < GR; ++gr) hmask[gr] = __builtin_amdgcn_ballot_w64(kap + 4 * gr < G);
    // token offset (within its block) of this lane's column in chunk rho
    int toff[4];
#pragma unroll
    for (int rho = 0; rho < 4; ++rho) {
        const int x = j16 & 7;
        const int g = x < 4 ? (rho == 0 ? 3 : rho - 1) : (rho == 0 ? 7 : rho + 3);
        toff[rho] = 32 * (j16 >> 3) + g + 8 * (x & 3);
    }
    // digit-tile read offset (block 0) of read r
    uint32_t arow[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) arow[r] = (uint32_t)(((32 * r + 8 * kap + (j16 >> 1)) * 2 + (j16 & 1)) * 8);

    // physical block of a logical one: runs of 2^rlog blocks, one run in every stride.
    // The NB blocks of an iteration lie in one run, so they are consecutive;
    // blocks past the index read as zeros (the buffer bound) and are masked.
    const int rlog = a.run_log2 ? a.run_log2 : kRunLog2;
    auto phys = [&](int lb) {
        return __builtin_amdgcn_readfirstlane(((lb >> rlog) * stride << rlog) + (lb & ((1 << rlog) - 1)));
    };
    // a physical block in a run that the sample stage took (staged filter: not read, no candidates)
    auto sampled = [&](int pb) { return STG && MODE == kFilter && ((pb >> rlog) & (skip - 1)) == 0; };
    // per-lane offset of plane s of step u; a plane the slot does not read
    // gets bit 31 set, which is out of range (kept in vector registers: a
    // per-plane lane mask would take scalar registers for the whole loop)
    uint32_t vo[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            vo[u][s] = trow[u] | (~(uint32_t)(s - tt[u]) & kOOB);
            asm volatile("" : "+v"(vo[u][s]));
        }
    auto voff = [&](int u, int s) { return vo[u][s]; };
    // blocks at or past the end of the index: their lanes read nothing from
    // here on (only the last iterations of a pair have such blocks)
    auto mask_dead = [&](int pb0) {
        if (pb0 + NB > nbk) {
            const uint32_t dead = tbk < nbk - pb0 ? 0u : kOOB;
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int s = 0; s < 4; ++s) vo[u][s] |= dead;
        }
    };

    // the products of block b of the current iteration (digits and codes in LDS)
    auto products = [&](int b, v4i (&kk)[GR], v4i (&o)[4][GR]) {
        v2i ac[GR][4];
#pragma unroll
        for (int gr = 0; gr < GR; ++gr)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                ac[gr][r] = r < C ? tr8(coef + gr * kCoefBytes, (uint32_t)(b * (S * 16)) + arow[r]) : (v2i){0, 0};
#pragma unroll
        for (int gr = 0; gr < GR; ++gr) kk[gr] = mfma_k(ac[gr], dcol, C);
        v2i bc[4][4];
#pragma unroll
        for (int rho = 0; rho < 4; ++rho)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                bc[rho][r] = r < C ? tr8(code, rd[r][(rho + 2 * (b >> 1)) & 3] + (uint32_t)(2 * b * kHalfBytes<C>))
                                   : (v2i){0, 0};
#pragma unroll
        for (int rho = 0; rho < 4; ++rho)
#pragma unroll
            for (int gr = 0; gr < GR; ++gr) o[rho][gr] = mfma_k(ac[gr], bc[rho], C);
    };
    // Screen, per tile rho: a token whose exact S passes has fl(hi) >= hv =
    // 2^(rho-1) (P - K) / 2^16 - bound(lo), with P = pred(th) 2^-zeta; hv is
    // a float lower bound of that.
    auto screen = [&](const v4i (&kk)[GR], int Eb, float (&hv)[GR][4]) {
#pragma unroll
        for (int gr = 0; gr < GR; ++gr) {
            const float phi = __builtin_ldexpf(pth[gr], sig[gr] - 15 - Eb);
            const float z = phi - (float)(kk[gr].z + kk[gr].w * 256);
            const float zf = z - lob - 4.0f - fabsf(z) * (1.0f / 262144.0f);
#pragma unroll
            for (int rho = 0; rho < 4; ++rho)
                hv[gr][rho] = __builtin_fmaf(zf, rho == 0 ? 0.5f : (float)(1 << (rho - 1)),
                                             -(lob * (float)(1 << rho) + 2.0f));
        }
    };

    // Loads run one iteration ahead, into the registers just consumed: the
    // scales are used (and the next ones requested) first, then each plane
    // word, replaced by the next iteration's as soon as it is extracted.
    // Every iteration issues the same 4 + 16 loads -- a plane that no slot
    // of a step reads is requested out of range, which costs no memory
    // access -- so the compiler's waits are exact: an iteration's first wait
    // covers its scales and the loads before them, and each plane word's
    // wait covers only that word and the loads issued before it.
    auto issue_scales = [&](int pb0, bool live, uint32_t (&sn)[4]) {
        const __amdgpu_buffer_rsrc_t rs = scale_rsrc(pb0, live);
#pragma unroll
        for (int k = 0; k < 4; ++k) sn[k] = __builtin_amdgcn_raw_buffer_load_b16(rs, srow[k], 0, 0);
    };
    uint32_t w[4][4] = {}, sc[4];
    int lb0 = lg0 + wave * NB;
    {
        const int pb0 = phys(lb0);
        mask_dead(pb0);
        const bool live0 = !sampled(pb0);
        const __amdgpu_buffer_rsrc_t r = plane_rsrc(pb0, live0);
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int s = 0; s < 4; ++s)
                w[u][s] = __builtin_amdgcn_raw_buffer_load_b32(r, voff(u, s), (int)(s * ldb8), 0);
        issue_scales(pb0, live0, sc);
    }
    for (; lb0 < lgend; lb0 += IB) {
        const int lbn = lb0 + IB;
        const bool more = lbn < lgend;
        const int pb0 = phys(lb0), pbn = more ? phys(lbn) : 0;  // past the end: zero records, nothing is read
        int nval[NB];  // valid tokens of block b (0 for dead blocks)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int64_t left = a.n - (int64_t)(pb0 + b) * 64;
            nval[b] = (lb0 + b < nlb && pb0 + b < nbk && !sampled(pb0)) ? (int)(left < 64 ? left : 64) : 0;
        }

        // ---- block exponents: largest exponent field of the read scales (>= 1);
        // fp16 bit patterns of non-negative values order like the values
        uint32_t mx = max(max(sc[0], sc[1]), max(sc[2], sc[3])) & 0xFFFFu;
        mx = max(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
        mx = max(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
        mx = max(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, 0x141, 0xF, 0xF, false));  // row_half_mirror
        mx = max(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, 0x140, 0xF, 0xF, false));  // row_mirror
        if (C >= 2) mx = max(mx, (uint32_t)__shfl_xor((int)mx, 16, kWave));
        if (C >= 4) mx = max(mx, (uint32_t)__shfl_xor((int)mx, 32, kWave));
        const int ef = max(1, (int)(mx >> 10) & 31);
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
                // scale 2^-(E+3): exact (a power of two times a binary16 value)
                const float sf = (float)__builtin_bit_cast(_Float16, (uint16_t)sc[k]) * pw;
#pragma unroll
                for (int gr = 0; gr < GR; ++gr) {
                    uint32_t dig[2];
#pragma unroll
                    for (int x = 0; x < 2; ++x) {
                        // trunc(fl32(q 2^sigma * scale) 2^-(E+3)): both power-of-two
                        // factors are exact, so this is that one rounding
                        const int Ai = (int)(qt[k][gr][x] * sf);
                        dig[x] = ((uint32_t)Ai + 0x00808080u) ^ 0x00808080u;
                    }
                    *(v2i*)(coef + gr * kCoefBytes + rb * (S * 16) + (e * 2 + rhp) * 8) =
                        (v2i){(int)dig[0], (int)dig[1]};
                }
            }
        }
        issue_scales(pbn, more && !sampled(pbn), sc);
        // ---- codes to LDS (a step with no slot to read writes nothing: its
        // stale records meet zero coefficients)
        if (more) mask_dead(pbn);
        const __amdgpu_buffer_rsrc_t rn = plane_rsrc(pbn, more && !sampled(pbn));
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            // the step's depth as a fresh scalar each iteration, so its
            // compares stay scalar branches instead of lane masks held (and
            // spilled) across the loop
            int tm = tmax[u];
            asm volatile("" : "+s"(tm));
            const bool act = tm != 0;  // wavefront-uniform
            v2i ch[4];
            if (act) extract(w[u], tm, ch);
#pragma unroll
            for (int s = 0; s < 4; ++s)
                w[u][s] = __builtin_amdgcn_raw_buffer_load_b32(rn, voff(u, s), (int)(s * ldb8), 0);
            if (act) {
#pragma unroll
                for (int rho = 0; rho < 4; ++rho)
                    *(v2i*)(code + wr[(rho + kSkewStep<C> * u) & 3] + u * 8 * C * kRec) = ch[rho];
            }
        }

        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // ---- products per block; block b+1's products are started before
        // block b is screened, so they run under its screen and staging
        v4i kkn[GR], on[4][GR];
        products(0, kkn, on);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int lb = lb0 + b;
            v4i kk[GR], o[4][GR];
#pragma unroll
            for (int gr = 0; gr < GR; ++gr) {
                kk[gr] = kkn[gr];
#pragma unroll
                for (int rho = 0; rho < 4; ++rho) o[rho][gr] = on[rho][gr];
            }
            if (b + 1 < NB) products(b + 1, kkn, on);
            if (MODE == kFilter) {
                float hv[GR][4];
                screen(kk, Eb[b], hv);
                // lanes whose (head, token) passes the screen, as wavefront masks
                uint64_t m[4][GR], mor = 0;
#pragma unroll
                for (int rho = 0; rho < 4; ++rho)
#pragma unroll
                    for (int gr = 0; gr < GR; ++gr) {
                        m[rho][gr] = __builtin_amdgcn_ballot_w64((float)(o[rho][gr].z + o[rho][gr].w * 256) >=
                                                                 hv[gr][rho]) & hmask[gr];
                        mor |= m[rho][gr];
                    }
                if (mor) {  // rare: the exact sums of the screened tokens go to the stage
                    if (nval[b] != 64) {  // the last block of a pair: drop its padding tokens
                        mor = 0;
#pragma unroll
                        for (int rho = 0; rho < 4; ++rho) {
                            const uint64_t vm = __builtin_amdgcn_ballot_w64(toff[rho] < nval[b]);
#pragma unroll
                            for (int gr = 0; gr < GR; ++gr) {
                                m[rho][gr] &= vm;
                                mor |= m[rho][gr];
                            }
                        }
                    }
#pragma unroll
                    for (int gr = 0; gr < GR; ++gr) {
                        const int64_t Kc = recombine(kk[gr]);
                        const uint32_t tag = (uint32_t)(kap + 4 * gr) | ((uint32_t)(Eb[b] - 1 - sig[gr]) << 16);
#pragma unroll
                        for (int rho = 0; rho < 4; ++rho) {
                            const uint64_t mm = m[rho][gr];
                            if (!mm) continue;
                            const uint32_t np = (uint32_t)__popcll(mm);
                            if (scnt + np > (uint32_t)kStage) flush();
                            if ((mm >> lane) & 1u) {
                                const int64_t x = recombine(o[rho][gr]);
                                const int64_t S = (rho == 0 ? x * 2 : (x >> (rho - 1))) + Kc;
                                const uint32_t tok = (uint32_t)(pb0 + b) * 64u + (uint32_t)toff[rho];
                                stage[scnt + (uint32_t)__popcll(mm & lanes_below(lane))] =
                                    (v4i){(int)(uint32_t)S, (int)(uint32_t)((uint64_t)S >> 32), (int)tok, (int)tag};
                            }
                            scnt += np;
                        }
                    }
                }
            } else {
                if (MODE == kStore || STG) {  // every score (LANEMAX, staged: into the second output)
                    float* const so = MODE == kStore ? a.out : a.out2;
#pragma unroll
                    for (int rho = 0; rho < 4; ++rho) {
                        const bool tval = toff[rho] < nval[b];
#pragma unroll
                        for (int gr = 0; gr < GR; ++gr) {
                            const int h = kap + 4 * gr;
                            const float sc = exact_score(o[rho][gr], recombine(kk[gr]), rho, Eb[b] - 1 - sig[gr]);
                            if (h < G && lb < nlb)
                                so[((size_t)op * G + h) * (a.nlb * 64) + (int64_t)lb * 64 + toff[rho]] =
                                    tval ? sc : -INFINITY;
                        }
                    }
                }
                if (MODE == kLaneMax) {
                    // Maxima of 16 tokens from the top two digit rows (S ~ 2^(17-rho)
                    // hi + K): the sample is only a statistic for the threshold, whose
                    // exactness the candidate count check keeps, so an estimate
                    // within a few units in 2^16 of the exact sum serves.
#pragma unroll
                    for (int gr = 0; gr < GR; ++gr) {
                        const float Kf = __builtin_fmaf((float)(kk[gr].z + kk[gr].w * 256), 65536.0f,
                                                        (float)(kk[gr].x + kk[gr].y * 256));
                        float v = -INFINITY;
#pragma unroll
                        for (int rho = 0; rho < 4; ++rho) {
                            const float e = __builtin_fmaf((float)(o[rho][gr].z + o[rho][gr].w * 256),
                                                           (float)(1 << (17 - rho)), Kf);
                            v = nval[b] == 64 || toff[rho] < nval[b] ? fmaxf(v, e) : v;
                        }
                        v = __builtin_ldexpf(v, Eb[b] - 1 - sig[gr]);
                        // lanes 4q .. 4q+3 of a head hold one group of 16 tokens
                        v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                         0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false)));  // quad_perm 1,0,3,2
                        v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                         0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false)));  // quad_perm 2,3,0,1
                        const int h = kap + 4 * gr;
                        if ((j16 & 3) == 0 && h < G && lb < nlb)
                            a.out[((size_t)op * G + h) * (a.nlb * 4) + (int64_t)lb * 4 + (j16 >> 2)] = v;
                    }
                }
            }
        }
        __builtin_amdgcn_wave_barrier();  // the next iteration rewrites this wavefront's LDS
    }
    if (MODE == kFilter && scnt) flush();
}

// The same tile with the plane loads shared out by slot (see the comment
// on the codes below): one 16-byte load per plane and lane covers every
// block of a workgroup iteration, so each line is requested once, at the
// price of two workgroup barriers per iteration.  It pays when the slot
// quarters are about equally deep (fixed-depth plans, and A > 64), and loses
// to the per-wavefront form when the deep slots sit in one quarter (the
// others wait for it at the barrier).
template <int GR, int MODE, int C, bool STG>
__device__ __forceinline__ void scan_body_shared(const ScanArgs& a, const int p, const int G, const int A,
                                          const int tile, const int op, const PairTables<GR>& T,
                                          unsigned char* code0, unsigned char* code, unsigned char* coef,
                                          v4i* stage)
{
    constexpr int S = 32 * C, NB = 4 / C;
    constexpr int NH = 4 * GR;
    constexpr int IB = kWaves * NB;  // logical blocks the workgroup takes per iteration
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    const int kap = lane >> 4, j16 = lane & 15;  // lane group (slot block / head) and row
    // block indices fit 32 bits (the host caps n below 2^31 tokens), and the
    // plane and scale offsets below fit 31 bits (the host rejects a pair whose
    // plane rows span 2^31 bytes or more)
    const int nlb = (int)a.nlb, nbk = (int)a.nb, stride = (int)a.stride, skip = (int)a.skip;
    // Iteration i of the workgroup reads the plane words of logical blocks
    // lg0 + i IB .. lg0 + i IB + IB - 1 (each wavefront its own slots), and
    // wavefront w multiplies and scores blocks lg0 + i IB + w NB + (0 .. NB-1).
    const int lg0 = tile * a.gb;
    const int lgend = min(lg0 + a.gb, nlb);
    const int64_t ldb = a.ldb;
    const uint32_t ldb8 = (uint32_t)(ldb * 8);

    // the pair's planes and scales; the descriptors are rebased on every
    // iteration's first physical block, so the range check stays exact
    const uint64_t* pplanes = a.planes + (size_t)p * a.D * 4 * ldb;
    const uint16_t* pscales = a.scales + (size_t)p * a.D * ldb;
    const uint32_t pbytes = (uint32_t)((int64_t)a.D * 4 * ldb * 8);
    const uint32_t sbytes = (uint32_t)((int64_t)a.D * ldb * 2);
    constexpr uint32_t kOOB = 0x80000000u;  // past every record: the load returns 0
    // (the record count is formed with a signed max: a saturating subtract
    // would be computed per lane and turn the descriptor into a per-lane value)
    auto records = [](uint32_t total, uint32_t off, bool live) {
        return __builtin_amdgcn_readfirstlane(live ? max((int)total - (int)off, 0) : 0);
    };
    // plane s of a row is read at the row's plane-0 offset (per lane) plus
    // s * ldb * 8 (the scalar offset); a lane whose block lies past the
    // index is pointed out of range (see `mask_dead`), so no read ever leaves
    // the pair's planes, whether or not the range check counts the scalar offset
    auto plane_rsrc = [&](int pb0, bool live) {
        const uint32_t off = (uint32_t)pb0 * 8u;
        return __builtin_amdgcn_make_buffer_rsrc((void*)((const unsigned char*)pplanes + off), (short)0,
                                                 records(pbytes, off, live), 0x00020000);
    };
    auto scale_rsrc = [&](int pb0, bool live) {
        const uint32_t off = (uint32_t)pb0 * 2u;
        return __builtin_amdgcn_make_buffer_rsrc((void*)((const unsigned char*)pscales + off), (short)0,
                                                 records(sbytes, off, live), 0x00020000);
    };

    // ---- codes.  The workgroup's IB blocks of an iteration are shared out
    // by slot: wavefront w extracts slots 8C w .. 8C w + 8C - 1 (its steps
    // C w .. C w + C - 1, deepest first) of all IB blocks, lane L taking
    // slot 8C w + L / (8/C) and the block pair 2 (L % (8/C)) + {0, 1}.  One
    // 16-byte load per plane then covers the row segments of all IB blocks
    // (a whole 128-byte line for C = 1), so each line is requested once;
    // the records are written where the wavefront that multiplies the block
    // reads them, behind a workgroup barrier.
    constexpr int LPR = 8 / C;  // lanes per row segment (block pairs per iteration)
    const int wsl = lane / LPR, wbp = lane % LPR;
    // which quarter of the slots this wavefront extracts: rotated from one
    // workgroup to the next, so that the deep slots (more planes) do not
    // always fall to the same wavefront position, i.e. the same SIMD
    const int wq = (wave + tile + p) & 3;
    const int we = 8 * C * wq + wsl;  // the lane's slot
    const int wt = (int)(T.slot[we] >> 8);
    const int wj = (int)(T.slot[we] & 255u);
    // the deepest slot of the quarter (slots are sorted deepest first)
    const int wtm = __builtin_amdgcn_readfirstlane((int)(T.slot[8 * C * wq] >> 8));
    // the lane's plane-3 row ends the pair's planes: a 16-byte read of its
    // last block pair would pass that end (see `mask_dead`)
    const bool wlast = wt == 4 && wj == a.D - 1;
    // record write offsets: record (block pair half i, half block hs) of the
    // lane, chunk rho, is at wr[rho] + i * kPairStep + hs * H in s_code
    constexpr uint32_t kPairStep = C == 4 ? (uint32_t)kCodeStride : 2u * (uint32_t)kHalfBytes<C>;
    uint32_t wr[4];
    {
        const int b0 = 2 * wbp, cw = b0 / NB, bl = b0 % NB;
        const int sk = rec_skew(we, bl);
        const uint32_t base = (uint32_t)(cw * kCodeStride + 2 * bl * kHalfBytes<C> + we * kRec);
#pragma unroll
        for (int m = 0; m < 4; ++m) wr[m] = base + (uint32_t)(((m + sk) & 3) * 8);
    }
    // transposing read offsets: read r of tile (b, rho) is rd[r][(rho + 2 (b/2)) & 3] + 2 b H
    uint32_t rd[C][4];
#pragma unroll
    for (int r = 0; r < C; ++r) {
        const int e = 32 * r + 8 * kap + (j16 >> 1), hs = j16 & 1;
        const int sk = rec_skew(e, 0);
        const uint32_t base = (uint32_t)(hs * kHalfBytes<C> + e * kRec);
#pragma unroll
        for (int m = 0; m < 4; ++m) rd[r][m] = base + (uint32_t)(((m + sk) & 3) * 8);
    }
    // ---- digit rows: the 16C lanes of block L / 16C compute its (slot,
    // head pair) rows pi = L % 16C + 16C k, k = 0..3 (slot pi / 2, pair L & 1)
    constexpr int LPB = 16 * C;
    const int rb = lane / LPB, rl = lane % LPB, rhp = lane & 1;
    uint32_t srow[4];  // scale byte offset of slot k from the iteration's first block (out of range past A)
    float qt[4][GR][2];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int e = (rl >> 1) + 8 * C * k;
        const int j = (int)(T.slot[e] & 255u);
        srow[k] = e < A ? (uint32_t)j * (uint32_t)(ldb * 2) + (uint32_t)rb * 2u : kOOB;
#pragma unroll
        for (int gr = 0; gr < GR; ++gr)
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const int h = 4 * gr + 2 * rhp + x;
                qt[k][gr][x] = (e < A && h < G)
                    ? __builtin_ldexpf(T.qv[h][j], T.sig[h]) : 0.0f;
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
    // FILTER: screened tokens wait in this wavefront's stage as (exact sum,
    // token, head | exponent << 16) records; a flush turns them into scores,
    // keeps those at or above their head's threshold, and appends them to the
    // candidate lists with one fetch-and-add per head
    uint32_t scnt = 0;  // wavefront-uniform
    auto flush = [&]() {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        for (uint32_t r0 = 0; r0 < scnt; r0 += kWave) {
            const bool valid = r0 + (uint32_t)lane < scnt;
            v4i rec = valid ? stage[r0 + lane] : (v4i){0, 0, 0, 0};
            const int h = rec.w & 0xFF, zeta = rec.w >> 16;
            const int64_t S = (int64_t)(((uint64_t)(uint32_t)rec.y << 32) | (uint32_t)rec.x);
            const float sc = (float)__builtin_ldexp((double)S, zeta);
            const bool keep = valid && sc >= T.thr[h];
            const uint64_t cv = composite(score_key(sc), (uint32_t)rec.z);
            uint32_t nh = 0, mine = 0;
            uint64_t mh[NH];
#pragma unroll
            for (int hh = 0; hh < NH; ++hh) {
                mh[hh] = __builtin_amdgcn_ballot_w64(keep && h == hh);
                if (lane == hh) nh = (uint32_t)__popcll(mh[hh]);
                if (h == hh) mine = (uint32_t)__popcll(mh[hh] & lanes_below(lane));
            }
            uint32_t base = 0;
            if (lane < NH && lane < G && nh) base = atomicAdd(&a.counts[(size_t)p * G + lane], nh);
            const uint32_t bh = (uint32_t)__shfl((int)base, h, kWave);
            if (keep && (int64_t)(bh + mine) < a.cap) a.cand[((size_t)p * G + h) * a.cap + bh + mine] = cv;
        }
        scnt = 0;
    };
    // lanes of existing heads, per head group
    uint64_t hmask[GR];
#pragma unroll
    for (int gr = 0; gr < GR; ++gr) hmask[gr] = __builtin_amdgcn_ballot_w64(kap + 4 * gr < G);
    // token offset (within its block) of this lane's column in chunk rho
    int toff[4];
#pragma unroll
    for (int rho = 0; rho < 4; ++rho) {
        const int x = j16 & 7;
        const int g = x < 4 ? (rho == 0 ? 3 : rho - 1) : (rho == 0 ? 7 : rho + 3);
        toff[rho] = 32 * (j16 >> 3) + g + 8 * (x & 3);
    }
    // digit-tile read offset (block 0) of read r
    uint32_t arow[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) arow[r] = (uint32_t)(((32 * r + 8 * kap + (j16 >> 1)) * 2 + (j16 & 1)) * 8);

    // physical block of a logical one: runs of 2^rlog blocks, one run in every stride.
    // The NB blocks of an iteration lie in one run, so they are consecutive;
    // blocks past the index read as zeros (the buffer bound) and are masked.
    const int rlog = a.run_log2 ? a.run_log2 : kRunLog2;
    auto phys = [&](int lb) {
        return __builtin_amdgcn_readfirstlane(((lb >> rlog) * stride << rlog) + (lb & ((1 << rlog) - 1)));
    };
    // a physical block in a run that the sample stage took (staged filter: not read, no candidates)
    auto sampled = [&](int pb) { return STG && MODE == kFilter && ((pb >> rlog) & (skip - 1)) == 0; };
    // per-lane offset of plane s of the lane's row segment; a plane the slot
    // does not read gets bit 31 set, which is out of range (kept in vector
    // registers: a per-plane lane mask would take scalar registers for the
    // whole loop)
    uint32_t vo[4];
    {
        const uint32_t row = wt ? (uint32_t)wj * 4u * ldb8 + (uint32_t)wbp * 16u : 0u;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            vo[s] = (row + (uint32_t)s * ldb8) | (~(uint32_t)(s - wt) & kOOB);
            asm volatile("" : "+v"(vo[s]));
        }
    }
    // Last iterations of a pair (the workgroup's base pw0 + IB past the
    // index): block pairs that lie wholly past the index read nothing; and a
    // 16-byte read of the pair's very last plane row at its last block would
    // cross the end of the pair's planes, where the range check drops the
    // whole read -- it is moved back 8 bytes (the block then sits in the
    // upper half, see `fix_shift`).  Blocks past the index in the other rows
    // read neighbouring memory of the pair and are masked by their token
    // counts.  Returns whether a lane was moved.
    bool shifted = false;
    auto mask_dead = [&](int pw0) {
        if (pw0 + IB > nbk) {
            const int fb = pw0 + 2 * wbp;  // the lane's first block
            const uint32_t dead = fb < nbk ? 0u : kOOB;
#pragma unroll
            for (int s = 0; s < 4; ++s) vo[s] |= dead;
            if (wlast && fb < nbk && fb + 1 >= (int)ldb) {
                vo[3] -= 8u;
                shifted = true;
            }
        }
    };
    auto fix_shift = [&](v4i (&w)[4]) {
        if (shifted) {
            w[3].x = w[3].z;
            w[3].y = w[3].w;
        }
    };
    // codes of the lane's four half blocks to LDS; plane s of record
    // (i, hs) is component 2 i + hs of w[s]
    auto codes_to_lds = [&](const v4i (&w)[4], unsigned char* code0) {
        if (wtm == 0) return;  // no slot of this wavefront is read: its stale records meet zero coefficients
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int hs = 0; hs < 2; ++hs) {
                const int c = 2 * i + hs;
                const uint32_t hw[4] = {(uint32_t)w[0][c], (uint32_t)w[1][c], (uint32_t)w[2][c],
                                        (uint32_t)w[3][c]};
                v2i ch[4];
                extract(hw, wtm, ch);
#pragma unroll
                for (int rho = 0; rho < 4; ++rho)
                    *(v2i*)(code0 + wr[rho] + i * kPairStep + hs * kHalfBytes<C>) = ch[rho];
            }
    };

    // the products of block b of the current iteration (digits and codes in LDS)
    auto products = [&](int b, v4i (&kk)[GR], v4i (&o)[4][GR]) {
        v2i ac[GR][4];
#pragma unroll
        for (int gr = 0; gr < GR; ++gr)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                ac[gr][r] = r < C ? tr8(coef + gr * kCoefBytes, (uint32_t)(b * (S * 16)) + arow[r]) : (v2i){0, 0};
#pragma unroll
        for (int gr = 0; gr < GR; ++gr) kk[gr] = mfma_k(ac[gr], dcol, C);
        v2i bc[4][4];
#pragma unroll
        for (int rho = 0; rho < 4; ++rho)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                bc[rho][r] = r < C ? tr8(code, rd[r][(rho + 2 * (b >> 1)) & 3] + (uint32_t)(2 * b * kHalfBytes<C>))
                                   : (v2i){0, 0};
#pragma unroll
        for (int rho = 0; rho < 4; ++rho)
#pragma unroll
            for (int gr = 0; gr < GR; ++gr) o[rho][gr] = mfma_k(ac[gr], bc[rho], C);
    };
    // Screen, per tile rho: a token whose exact S passes has fl(hi) >= hv =
    // 2^(rho-1) (P - K) / 2^16 - bound(lo), with P = pred(th) 2^-zeta; hv is
    // a float lower bound of that.
    auto screen = [&](const v4i (&kk)[GR], int Eb, float (&hv)[GR][4]) {
#pragma unroll
        for (int gr = 0; gr < GR; ++gr) {
            const float phi = __builtin_ldexpf(pth[gr], sig[gr] - 15 - Eb);
            const float z = phi - (float)(kk[gr].z + kk[gr].w * 256);
            const float zf = z - lob - 4.0f - fabsf(z) * (1.0f / 262144.0f);
#pragma unroll
            for (int rho = 0; rho < 4; ++rho)
                hv[gr][rho] = __builtin_fmaf(zf, rho == 0 ? 0.5f : (float)(1 << (rho - 1)),
                                             -(lob * (float)(1 << rho) + 2.0f));
        }
    };

    // Loads run one iteration ahead, into the registers just consumed: the
    // scales are used (and the next ones requested) first, then the plane
    // words once their codes are in LDS.  Every iteration issues the same
    // 4 + 4 loads -- a plane that the lane's slot does not read is requested
    // out of range, which costs no memory access -- so the compiler's waits
    // are exact.
    auto issue_scales = [&](int pb0, bool live, uint32_t (&sn)[4]) {
        const __amdgpu_buffer_rsrc_t rs = scale_rsrc(pb0, live);
#pragma unroll
        for (int k = 0; k < 4; ++k) sn[k] = __builtin_amdgcn_raw_buffer_load_b16(rs, srow[k], 0, 0);
    };
    v4i w[4];
    uint32_t sc[4];
    {
        const int pw0 = phys(lg0);
        mask_dead(pw0);
        const bool live0 = !sampled(pw0);
        const __amdgpu_buffer_rsrc_t r = plane_rsrc(pw0, live0);
#pragma unroll
        for (int s = 0; s < 4; ++s) w[s] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, vo[s], 0, 0));
        issue_scales(phys(lg0 + wave * NB), live0, sc);
    }
    for (int lw0 = lg0; lw0 < lgend; lw0 += IB) {
        const int lb0 = lw0 + wave * NB;  // this wavefront's blocks (products, scales, outputs)
        const bool more = lw0 + IB < lgend;
        const bool tail = phys(lw0) + IB > nbk;  // blocks past the index (see `mask_dead`)
        const int pb0 = phys(lb0), pbn = more ? phys(lb0 + IB) : 0;  // past the end: zero records, nothing is read
        const int pwn = more ? phys(lw0 + IB) : 0;
        int nval[NB];  // valid tokens of block b (0 for dead blocks)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int64_t left = a.n - (int64_t)(pb0 + b) * 64;
            nval[b] = (lb0 + b < nlb && pb0 + b < nbk && !sampled(pb0)) ? (int)(left < 64 ? left : 64) : 0;
        }

        // ---- block exponents: largest exponent field of the read scales (>= 1);
        // fp16 bit patterns of non-negative values order like the values
        uint32_t mx = max(max(sc[0], sc[1]), max(sc[2], sc[3])) & 0xFFFFu;
        mx = max(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
        mx = max(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
        mx = max(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, 0x141, 0xF, 0xF, false));  // row_half_mirror
        mx = max(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, 0x140, 0xF, 0xF, false));  // row_mirror
        if (C >= 2) mx = max(mx, (uint32_t)__shfl_xor((int)mx, 16, kWave));
        if (C >= 4) mx = max(mx, (uint32_t)__shfl_xor((int)mx, 32, kWave));
        const int ef = max(1, (int)(mx >> 10) & 31);
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
                // scale 2^-(E+3): exact (a power of two times a binary16 value)
                const float sf = (float)__builtin_bit_cast(_Float16, (uint16_t)sc[k]) * pw;
#pragma unroll
                for (int gr = 0; gr < GR; ++gr) {
                    uint32_t dig[2];
#pragma unroll
                    for (int x = 0; x < 2; ++x) {
                        // trunc(fl32(q 2^sigma * scale) 2^-(E+3)): both power-of-two
                        // factors are exact, so this is that one rounding
                        const int Ai = (int)(qt[k][gr][x] * sf);
                        dig[x] = ((uint32_t)Ai + 0x00808080u) ^ 0x00808080u;
                    }
                    *(v2i*)(coef + gr * kCoefBytes + rb * (S * 16) + (e * 2 + rhp) * 8) =
                        (v2i){(int)dig[0], (int)dig[1]};
                }
            }
        }
        issue_scales(pbn, more && !sampled(pbn), sc);
        // ---- codes to LDS, then the next iteration's plane words
        if (tail) fix_shift(w);
        if (wq == 0) __builtin_amdgcn_s_setprio(3);  // the deepest slots: the others wait on it
        codes_to_lds(w, code0);
        shifted = false;
        if (more) mask_dead(pwn);
        {
            const __amdgpu_buffer_rsrc_t rn = plane_rsrc(pwn, more && !sampled(pwn));
#pragma unroll
            for (int s = 0; s < 4; ++s)
                w[s] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rn, vo[s], 0, 0));
        }
        __syncthreads();  // every wavefront's records (and digit rows) are in LDS
        __builtin_amdgcn_s_setprio(0);

        // ---- products per block; block b+1's products are started before
        // block b is screened, so they run under its screen and staging
        v4i kkn[GR], on[4][GR];
        products(0, kkn, on);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int lb = lb0 + b;
            v4i kk[GR], o[4][GR];
#pragma unroll
            for (int gr = 0; gr < GR; ++gr) {
                kk[gr] = kkn[gr];
#pragma unroll
                for (int rho = 0; rho < 4; ++rho) o[rho][gr] = on[rho][gr];
            }
            if (b + 1 < NB) products(b + 1, kkn, on);
            if (MODE == kFilter) {
                float hv[GR][4];
                screen(kk, Eb[b], hv);
                // lanes whose (head, token) passes the screen, as wavefront masks
                uint64_t m[4][GR], mor = 0;
#pragma unroll
                for (int rho = 0; rho < 4; ++rho)
#pragma unroll
                    for (int gr = 0; gr < GR; ++gr) {
                        m[rho][gr] = __builtin_amdgcn_ballot_w64((float)(o[rho][gr].z + o[rho][gr].w * 256) >=
                                                                 hv[gr][rho]) & hmask[gr];
                        mor |= m[rho][gr];
                    }
                if (mor) {  // rare: the exact sums of the screened tokens go to the stage
                    if (nval[b] != 64) {  // the last block of a pair: drop its padding tokens
                        mor = 0;
#pragma unroll
                        for (int rho = 0; rho < 4; ++rho) {
                            const uint64_t vm = __builtin_amdgcn_ballot_w64(toff[rho] < nval[b]);
#pragma unroll
                            for (int gr = 0; gr < GR; ++gr) {
                                m[rho][gr] &= vm;
                                mor |= m[rho][gr];
                            }
                        }
                    }
#pragma unroll
                    for (int gr = 0; gr < GR; ++gr) {
                        const int64_t Kc = recombine(kk[gr]);
                        const uint32_t tag = (uint32_t)(kap + 4 * gr) | ((uint32_t)(Eb[b] - 1 - sig[gr]) << 16);
#pragma unroll
                        for (int rho = 0; rho < 4; ++rho) {
                            const uint64_t mm = m[rho][gr];
                            if (!mm) continue;
                            const uint32_t np = (uint32_t)__popcll(mm);
                            if (scnt + np > (uint32_t)kStage) flush();
                            if ((mm >> lane) & 1u) {
                                const int64_t x = recombine(o[rho][gr]);
                                const int64_t S = (rho == 0 ? x * 2 : (x >> (rho - 1))) + Kc;
                                const uint32_t tok = (uint32_t)(pb0 + b) * 64u + (uint32_t)toff[rho];
                                stage[scnt + (uint32_t)__popcll(mm & lanes_below(lane))] =
                                    (v4i){(int)(uint32_t)S, (int)(uint32_t)((uint64_t)S >> 32), (int)tok, (int)tag};
                            }
                            scnt += np;
                        }
                    }
                }
            } else {
                if (MODE == kStore || STG) {  // every score (LANEMAX, staged: into the second output)
                    float* const so = MODE == kStore ? a.out : a.out2;
#pragma unroll
                    for (int rho = 0; rho < 4; ++rho) {
                        const bool tval = toff[rho] < nval[b];
#pragma unroll
                        for (int gr = 0; gr < GR; ++gr) {
                            const int h = kap + 4 * gr;
                            const float sc = exact_score(o[rho][gr], recombine(kk[gr]), rho, Eb[b] - 1 - sig[gr]);
                            if (h < G && lb < nlb)
                                so[((size_t)op * G + h) * (a.nlb * 64) + (int64_t)lb * 64 + toff[rho]] =
                                    tval ? sc : -INFINITY;
                        }
                    }
                }
                if (MODE == kLaneMax) {
                    // Maxima of 16 tokens from the top two digit rows (S ~ 2^(17-rho)
                    // hi + K): the sample is only a statistic for the threshold, whose
                    // exactness the candidate count check keeps, so an estimate
                    // within a few units in 2^16 of the exact sum serves.
#pragma unroll
                    for (int gr = 0; gr < GR; ++gr) {
                        const float Kf = __builtin_fmaf((float)(kk[gr].z + kk[gr].w * 256), 65536.0f,
                                                        (float)(kk[gr].x + kk[gr].y * 256));
                        float v = -INFINITY;
#pragma unroll
                        for (int rho = 0; rho < 4; ++rho) {
                            const float e = __builtin_fmaf((float)(o[rho][gr].z + o[rho][gr].w * 256),
                                                           (float)(1 << (17 - rho)), Kf);
                            v = nval[b] == 64 || toff[rho] < nval[b] ? fmaxf(v, e) : v;
                        }
                        v = __builtin_ldexpf(v, Eb[b] - 1 - sig[gr]);
                        // lanes 4q .. 4q+3 of a head hold one group of 16 tokens
                        v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                         0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false)));  // quad_perm 1,0,3,2
                        v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                         0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false)));  // quad_perm 2,3,0,1
                        const int h = kap + 4 * gr;
                        if ((j16 & 3) == 0 && h < G && lb < nlb)
                            a.out[((size_t)op * G + h) * (a.nlb * 4) + (int64_t)lb * 4 + (j16 >> 2)] = v;
                    }
                }
            }
        }
        __syncthreads();  // the records are read: the next iteration rewrites them
    }
    if (MODE == kFilter && scnt) flush();
}

template <int GR, int MODE, bool STG>
__device__ __forceinline__ void scan_pair(const ScanArgs& a, const int p, const int G, const int tile,
                                          const int op)
{
    constexpr int NH = 4 * GR;
    __shared__ PairTables<GR> T;
    __shared__ __attribute__((aligned(16))) unsigned char s_code[kWaves][kCodeStride];
    __shared__ __attribute__((aligned(16))) unsigned char s_coef[kWaves][GR * kCoefBytes];
    __shared__ v4i s_stage[MODE == kFilter ? kWaves : 1][MODE == kFilter ? kStage : 1];

    const int lane = lane_id(), wave = threadIdx.x / kWave;
    const int A = a.n_active[p];

    // ---- pair tables: slots sorted by depth (counting sort), scaled queries.
    // Every global value the tables need is requested at once (the active
    // list, the channels' depths, the heads' query values, the thresholds),
    // so a workgroup's set-up waits for one round trip to memory; the rest
    // works in LDS.
    uint32_t tk = 0;
    if (MODE == kFilter && (int)threadIdx.x < G) tk = a.tau[(size_t)p * G + threadIdx.x];
    for (int e = threadIdx.x; e < a.D; e += kThreads) {
        T.act[e] = a.active[(size_t)p * a.D + e];  // entries past A are read but not used
        T.tch[e] = (unsigned char)a.depth[(size_t)p * a.D + e];
        for (int h = 0; h < G && h < NH; ++h) T.qv[h][e] = a.q_used[((size_t)p * G + h) * a.D + e];
    }
    if (threadIdx.x < 5) T.cnt[threadIdx.x] = 0u;
    if (threadIdx.x < NH) T.qmax[threadIdx.x] = 0u;
    __syncthreads();
    for (int e = threadIdx.x; e < A; e += kThreads) {
        const int j = T.act[e];
        atomicAdd(&T.cnt[T.tch[j]], 1u);
        for (int h = 0; h < G && h < NH; ++h)  // |q| bits order like |q| values
            atomicMax(&T.qmax[h], __float_as_uint(fabsf(T.qv[h][j])));
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
        float th = INFINITY;
        if (MODE == kFilter && (int)threadIdx.x < G) th = tk <= 0x007FFFFFu ? -INFINITY : key_score(tk);
        T.thr[threadIdx.x] = th;
    }
    __syncthreads();
    if (wave == 0) {  // slots of a depth class in ascending channel order
        for (int e0 = 0; e0 < A; e0 += kWave) {
            const int e = e0 + lane;
            int j = 0, t = 0;
            if (e < A) {
                j = T.act[e];
                t = T.tch[j];
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
    v4i* stage = s_stage[MODE == kFilter ? wave : 0];
    // the four slot quarters equally deep (the deepest slot of the last
    // quarter as deep as the first), or A > 64: loads shared out by slot
    const int C = A <= 32 ? 1 : A <= 64 ? 2 : 4;
    const bool shared = C == 4 || (T.slot[0] >> 8) == (T.slot[24 * C] >> 8);
    if (shared) {
        if (C == 1) scan_body_shared<GR, MODE, 1, STG>(a, p, G, A, tile, op, T, s_code[0], code, coef, stage);
        else if (C == 2) scan_body_shared<GR, MODE, 2, STG>(a, p, G, A, tile, op, T, s_code[0], code, coef, stage);
        else scan_body_shared<GR, MODE, 4, STG>(a, p, G, A, tile, op, T, s_code[0], code, coef, stage);
    } else {
        if (C == 1) scan_body<GR, MODE, 1, STG>(a, p, G, A, tile, op, T, code, coef, stage);
        else scan_body<GR, MODE, 2, STG>(a, p, G, A, tile, op, T, code, coef, stage);
    }
}

// blockIdx.y is the pair, blockIdx.x its tile of gb logical blocks.
// STG: FILTER skips the runs the sample took (a.skip); LANEMAX also
// writes every score of the sample to a.out2.
template <int GR, int MODE, bool STG>
__global__ __launch_bounds__(kThreads) void scan_kernel(ScanArgs a, int G)
{
    scan_pair<GR, MODE, STG>(a, (int)blockIdx.y, G, (int)blockIdx.x, (int)blockIdx.y);
}

// Fused path, stage 3: the heads whose candidate list failed (more than
// cap candidates, or fewer than k) are selected over a full score row of
// their pair instead.  Failed pairs are numbered in pair order.

// Whether selection m failed.
__device__ __forceinline__ bool sel_failed(const uint32_t* counts, int64_t m, int64_t cap, int k)
{
    const int64_t c = counts[m];
    return c > cap || c < (int64_t)k;
}

// The pair numbered `nth` among the failed ones, or -1; every thread of the
// workgroup gets the same answer.
__device__ int nth_failed_pair(const uint32_t* __restrict__ counts, int P, int G, int64_t cap, int k,
                               uint32_t nth)
{
    __shared__ uint32_t s_wsum[kWaves];
    __shared__ int s_pair;
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    __syncthreads();  // a previous call's readers of s_pair and s_wsum are done
    if (threadIdx.x == 0) s_pair = -1;
    uint32_t seen = 0;  // failed pairs before this chunk
    for (int p0 = 0; p0 < P; p0 += kThreads) {
        const int p = p0 + (int)threadIdx.x;
        bool f = false;
        if (p < P)
            for (int h = 0; h < G; ++h) f |= sel_failed(counts, (int64_t)p * G + h, cap, k);
        const uint64_t b = __ballot(f);
        if (lane == 0) s_wsum[wave] = (uint32_t)__popcll(b);
        __syncthreads();
        uint32_t off = 0, nf = 0;
        for (int w = 0; w < kWaves; ++w) {
            off += w < wave ? s_wsum[w] : 0u;
            nf += s_wsum[w];
        }
        if (f && seen + off + (uint32_t)__popcll(b & lanes_below(lane)) == nth) s_pair = p;
        __syncthreads();
        const int r = s_pair;
        if (r >= 0 || nth < seen + nf) return r;
        seen += nf;
        __syncthreads();  // s_wsum is rewritten by the next chunk
    }
    return -1;
}

// (1) Failed pair number r (r < rows) is rescanned into score row r, tile
// blockIdx.x of it per workgroup, as fast as a scan of that many pairs.
template <int GR>
__global__ __launch_bounds__(kThreads) void repair_scan_kernel(ScanArgs a, int P, int G, int k,
                                                               const uint32_t* __restrict__ counts,
                                                               int64_t cap)
{
    const int fp = nth_failed_pair(counts, P, G, cap, k, blockIdx.y);
    if (fp < 0) return;
    scan_pair<GR, kStore, false>(a, fp, G, (int)blockIdx.x, (int)blockIdx.y);
}

// (2) Workgroup r selects the failed heads of failed pair r from row r
// (filled by (1)); then it takes failed pairs r + rows, r + 2 rows, ...,
// should there be more than rows of them, rescanning each whole pair
// itself into its row.  The rows bound the workspace whatever the number
// of failures; only failures beyond the first `rows` pairs are slow.
template <int GR>
__global__ __launch_bounds__(kThreads) void repair_select_kernel(ScanArgs a, int P, int G, int k,
                                                                 const uint32_t* __restrict__ counts,
                                                                 int64_t cap, int32_t* __restrict__ topk_idx,
                                                                 float* __restrict__ topk_val,
                                                                 int32_t* __restrict__ sorted_idx)
{
    __shared__ SelShared sh;
    const int64_t npad = a.nlb * 64;
    float* row = a.out + (size_t)blockIdx.x * G * npad;
    for (uint32_t i = blockIdx.x;; i += gridDim.x) {
        const int fp = nth_failed_pair(counts, P, G, cap, k, i);
        if (fp < 0) break;
        if (i >= gridDim.x) {
            scan_pair<GR, kStore, false>(a, fp, G, 0, (int)blockIdx.x);  // one tile: a.gb covers the pair
            __syncthreads();  // the row is complete (and the pair's LDS tables free)
        }
        for (int h = 0; h < G; ++h) {
            const int64_t m = (int64_t)fp * G + h;
            if (!sel_failed(counts, m, cap, k)) continue;
            select_one(row + (size_t)h * npad, a.n, npad, true, nullptr, 0, k, m, topk_idx, topk_val,
                       sorted_idx, sh);
            __syncthreads();  // sh is reused by the next head
        }
    }
}

template <int MODE>
hipError_t launch_mode(const ScanArgs& args, int P, int G, hipStream_t st)
{
    ScanArgs a = args;
    const int rows = P;
    // blocks per workgroup: 1024, or fewer (a multiple of every iteration's
    // 16 blocks, at least 64; see below for few pairs and the staged sample)
    // while the grid has fewer workgroups than
    // `target`.  Long ranges spread each workgroup's start-up (the pair's
    // tables, the first loads, the last flush) over more blocks: at 1M
    // tokens x 288 pairs the filtered scan takes 1.10 ms with 256 blocks per
    // workgroup, 0.98 with 512, 0.96 with 1024 and 1.00 with 2048.  For the
    // full scans of few pairs a grid of about two workgroups per CU does
    // well: at 1M tokens x 8 pairs (one layer) the filter takes 110 us with
    // 2048 workgroups of 64 blocks, 77 with 1024, 56 with 512 and 64 with
    // 256 (and 54.7 with the 632 of 208 blocks the rule below picks; 60.8
    // with 552, 57.3 with 752).  Many pairs of shorter rows want the
    // larger grid: at 131k tokens x 288 pairs 2304 workgroups of 256 blocks
    // filter in 0.19 ms against 0.22 for 576 of 1024.  The sampled stage
    // reads one run in 16, so its workgroups are short and more of them
    // (2048) keep the chip busy: 0.105 ms at 288 pairs against 0.125 with 512.
    // The staged sample of an index read over the host link (a.out2 set,
    // runs of 512 blocks) wants about 512 long workgroups, down to 32
    // blocks for few pairs: at 1M tokens x 288 pairs 3.67 ms with 576 of
    // 512 blocks against 3.83 with 32-block ones (and 3.97 for runs of 32).
    // Calls of few pairs (a layer's 8 KV heads) are latency-bound: a
    // workgroup's start-up (tables, first loads, last flush) costs about as
    // much as several iterations, so their grids aim at one round of
    // workgroups.  The sampled stage may go down to 16-block (one-iteration)
    // workgroups; the filter takes about 640 workgroups (2.5 per CU), or one
    // per CU where that would leave fewer than 64 blocks each.  One layer at
    // 1M tokens: sample 27 -> 23 us, filter 56.5 -> 54.7 us; the 36-layer
    // step 4.18 -> 3.96 ms, at 131k 3.47 -> 3.27 ms, the 32k step 95 -> 83 us.
    // Over the host link (the staged filter, a.skip set) longer workgroups
    // read faster, so that filter keeps the halving rule (36 layers at 1M:
    // 55.0 ms against 57.0 with the few-pairs grid).
    const bool host_sample = MODE == kLaneMax && a.out2 != nullptr;
    const int64_t target = host_sample ? 512 : MODE == kLaneMax || rows >= 64 ? 2048 : 512;
    const int floor_gb = host_sample ? 32 : (MODE == kLaneMax || (MODE == kStore && rows < 64)) ? 16 : 64;
    a.gb = kGroupBlocks;
    while (a.gb > floor_gb && (int64_t)((a.nlb + a.gb - 1) / a.gb) * rows < target) a.gb /= 2;
    if (MODE == kFilter && rows < 64 && a.skip == 0) {
        const int64_t work = a.nlb * rows;
        int64_t g = ((work + 639) / 640 + 15) / 16 * 16;
        if (g < 64) g = ((work + 255) / 256 + 15) / 16 * 16;
        a.gb = (int)(g < 16 ? 16 : g > kGroupBlocks ? kGroupBlocks : g);
    }
    dim3 grid((unsigned)((a.nlb + a.gb - 1) / a.gb), (unsigned)rows);
    const bool stg = (MODE == kFilter && a.skip != 0) || (MODE == kLaneMax && a.out2 != nullptr);
    if (MODE != kStore && stg) {
        // The staged filter reads over the host link; one workgroup per CU
        // (64 KB of otherwise unused LDS on top of the tables and stages)
        // keeps fewer rows of the mapped index in flight and reads faster
        // where the grid takes many rounds anyway: 47.3 -> 46.6 ms at 1M
        // tokens x 288 pairs (46.9 with two per CU).
        const size_t dyn = MODE == kFilter && (int64_t)grid.x * grid.y >= 2048 ? 65536 : 0;
        if (G <= 4) scan_kernel<1, MODE, MODE != kStore><<<grid, kThreads, dyn, st>>>(a, G);
        else scan_kernel<2, MODE, MODE != kStore><<<grid, kThreads, dyn, st>>>(a, G);
    } else {
        if (G <= 4) scan_kernel<1, MODE, false><<<grid, kThreads, 0, st>>>(a, G);
        else scan_kernel<2, MODE, false><<<grid, kThreads, 0, st>>>(a, G);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_scan_args(const ScanArgs& a, int P, int G, int mode, hipStream_t st)
{
    if (mode == kFilter) return launch_mode<kFilter>(a, P, G, st);
    if (mode == kLaneMax) return launch_mode<kLaneMax>(a, P, G, st);
    return launch_mode<kStore>(a, P, G, st);
}

hipError_t launch_repair(const ScanArgs& base, int P, int G, int k, const uint32_t* counts, int64_t cap,
                         float* rows, int slots, int32_t* topk_idx, float* topk_val, int32_t* sorted_idx,
                         hipStream_t st)
{
    ScanArgs a = base;
    a.stride = 1;
    a.nlb = a.nb;
    a.out = rows;
    // (1): tiles of the first `slots` failed pairs, sized like a scan of
    // that many pairs; workgroups of absent failures return at once
    a.gb = kGroupBlocks;
    while (a.gb > 64 && (int64_t)((a.nlb + a.gb - 1) / a.gb) * slots < 512) a.gb /= 2;
    const dim3 g1((unsigned)((a.nlb + a.gb - 1) / a.gb), (unsigned)slots);
    if (G <= 4) repair_scan_kernel<1><<<g1, kThreads, 0, st>>>(a, P, G, k, counts, cap);
    else repair_scan_kernel<2><<<g1, kThreads, 0, st>>>(a, P, G, k, counts, cap);
    // (2): selection, and one workgroup per row for any further failures
    a.gb = (int)a.nb;
    const dim3 g2((unsigned)slots);
    if (G <= 4) repair_select_kernel<1><<<g2, kThreads, 0, st>>>(a, P, G, k, counts, cap, topk_idx, topk_val, sorted_idx);
    else repair_select_kernel<2><<<g2, kThreads, 0, st>>>(a, P, G, k, counts, cap, topk_idx, topk_val, sorted_idx);
    return hipGetLastError();
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

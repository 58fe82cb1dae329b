/*
 * Fathom CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, single-threaded C for what the decode-step key scan computes.
 * Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may load
 * this library; the product path (sparse_attention_key_amd) never does.  It
 * shares no code, header, table or constant with the HIP library.
 *
 * Source: "Fathom: Per-Query Read Depth for Sparse Decoding over Offloaded KV
 * Caches" (arXiv 2609.17652) as described on the yeyulingfeng.com write-up
 * (sections "方法一: 把 K 缓存变成 bit plane", "方法二: 每个 query 组做一次反向注水",
 * "基座选择") and the paotong.dev bit-plane figure.  The page lost its formulas;
 * the readings used here are listed next to each function.
 *
 * Every function handles ONE (layer, KV head) pair.  Layouts:
 *   keys    [n][D]          float32, token-major
 *   planes  [D][4][nb]      uint64, plane s of channel j holds code bit (3-s),
 *                           bit i of word (j,s,b) = token 64*b+i
 *   scales  [D][nb]         IEEE binary16 bit patterns (block max |x|)
 *   q       [G][D]          float32
 *   scores  [G][nb*64]      float32 (tokens >= n are -inf)
 *
 * Parity status per function is stated in its comment; every function here is
 * pinned by tests/test_oracle_pins.py (none is "parity unpinned").
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_PLAN_WATERFILL 0
#define ORC_PLAN_TOPR 1
#define ORC_PLAN_UNIFORM 2

/* ---------------------------------------------------------------- binary16 */

/* float32 -> binary16, round to nearest, ties to even, from the IEEE 754
 * definition: values are exact in double, so the rounding is done on the
 * integer multiple of the target quantum.  |x| >= 65520 gives +-inf. */
uint16_t orc_f32_to_f16(float x)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    double a = fabs((double)x);
    if (isnan(x)) return 0x7E00u;
    if (a >= 65520.0) return (uint16_t)(sign | 0x7C00u);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e); /* a = f * 2^e, f in [0.5, 1): unbiased exponent e-1 */
    int ue = e - 1;
    double quantum = (ue < -14) ? ldexp(1.0, -24) : ldexp(1.0, ue - 10);
    double r = nearbyint(a / quantum); /* default mode: ties to even */
    double v = r * quantum;
    if (v == 0.0) return sign;
    if (v < ldexp(1.0, -14)) /* subnormal */
        return (uint16_t)(sign | (uint16_t)(v / ldexp(1.0, -24)));
    frexp(v, &e); /* rounding may have carried into the next binade */
    ue = e - 1;
    uint32_t mant = (uint32_t)(v / ldexp(1.0, ue - 10)) - 1024u;
    return (uint16_t)(sign | (uint16_t)((ue + 15) << 10) | mant);
}

float orc_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int ex = (h >> 10) & 31;
    int man = h & 1023;
    double v;
    if (ex == 31) v = man ? NAN : INFINITY;
    else if (ex == 0) v = ldexp((double)man, -24);
    else v = ldexp((double)(1024 + man), ex - 25);
    return (float)(sign ? -v : v);
}

/* ------------------------------------------------------------ quantisation */

/* Reading of the lost quantiser formula (method section one): per (64-token
 * block, channel) the block max m = max|x| is kept as an fp16 scale, the cell
 * width is scale/8, and the 4-bit code is c = clamp(floor(x / (scale/8)) + 8,
 * 0, 15): code 8 is the cell that starts at zero, the MSB is the sign.  The
 * floor is the exact real floor (double division of an fp32 by an
 * fp16-derived value never rounds across an integer).  A zero scale gives
 * code 8.  A scale that would overflow fp16 saturates to 65504. */
int orc_code(float x, uint16_t scale_bits)
{
    float scale = orc_f16_to_f32(scale_bits);
    float delta = scale * 0.125f; /* exact */
    if (!(delta > 0.0f)) return 8;
    double f = floor((double)x / (double)delta) + 8.0;
    if (f < 0.0) f = 0.0;
    if (f > 15.0) f = 15.0;
    return (int)f;
}

/* y_j = sum_d rot[d][j] * x_d as an fp32 fused multiply-add chain over
 * ascending d (the stored coordinates of the rotated basis, "基座选择"). */
static void rotate_row(const float* x, const float* rot, int D, float* y)
{
    for (int j = 0; j < D; ++j) {
        float acc = 0.0f;
        for (int d = 0; d < D; ++d) acc = fmaf(rot[(size_t)d * D + j], x[d], acc);
        y[j] = acc;
    }
}

/* Pack keys into channel-major bit planes plus per-block fp16 scales
 * (method section one; the paotong.dev plane figure).  Padding tokens of the
 * last block get code 8 and do not enter the block max. */
void orc_pack(const float* keys, int64_t n, int D, const float* rot, uint64_t* planes,
              uint16_t* scales)
{
    int64_t nb = (n + 63) / 64;
    float* blk = (float*)malloc(sizeof(float) * 64 * (size_t)D);
    memset(planes, 0, sizeof(uint64_t) * (size_t)D * 4 * (size_t)nb);
    for (int64_t b = 0; b < nb; ++b) {
        int valid = (int)((n - 64 * b) < 64 ? (n - 64 * b) : 64);
        for (int i = 0; i < valid; ++i) {
            const float* x = keys + (size_t)(64 * b + i) * D;
            if (rot) rotate_row(x, rot, D, blk + (size_t)i * D);
            else memcpy(blk + (size_t)i * D, x, sizeof(float) * D);
        }
        for (int j = 0; j < D; ++j) {
            float m = 0.0f;
            for (int i = 0; i < valid; ++i) {
                float a = fabsf(blk[(size_t)i * D + j]);
                if (a > m) m = a;
            }
            uint16_t sb = orc_f32_to_f16(m);
            if (sb == 0x7C00u) sb = 0x7BFFu; /* saturate */
            scales[(size_t)j * nb + b] = sb;
            for (int i = 0; i < 64; ++i) {
                int c = (i < valid) ? orc_code(blk[(size_t)i * D + j], sb) : 8;
                for (int s = 0; s < 4; ++s)
                    if ((c >> (3 - s)) & 1)
                        planes[((size_t)j * 4 + s) * nb + b] |= (uint64_t)1 << i;
            }
        }
    }
    free(blk);
}

/* Read the t-plane prefix of token i, channel j: c_t = c >> (4 - t). */
int orc_prefix_code(const uint64_t* planes, int64_t nb, int j, int64_t i, int t)
{
    int64_t b = i / 64;
    int bit = (int)(i % 64);
    int c = 0;
    for (int s = 0; s < t; ++s)
        c = (c << 1) | (int)((planes[((size_t)j * 4 + s) * nb + b] >> bit) & 1u);
    return c;
}

/* Dequantised t-bit prefix (method section one): the t-bit mid-rise
 * quantiser on [-scale, scale] with cell width 2^(4-t) * scale/8:
 *   k = (c_t - 2^(t-1) + 1/2) * 2^(4-t) * scale/8 = (2 c_t + 1 - 2^t) * 2^-t * scale.
 * Exact in fp32 (at most 4 significant bits times an fp16 mantissa).
 * t = 0 reads nothing and contributes 0. */
float orc_dequant(int ct, int t, uint16_t scale_bits)
{
    if (t == 0) return 0.0f;
    double odd = (double)(2 * ct + 1 - (1 << t));
    return (float)(odd * ldexp((double)orc_f16_to_f32(scale_bits), -t));
}

/* ------------------------------------------------------------------- plan */

/* Query used for scoring: q itself, or rot^T q (each output an fp32 fma
 * chain over ascending d) when keys are stored in the rotated basis. */
void orc_query_used(const float* q, const float* rot, int G, int D, float* q_used)
{
    for (int h = 0; h < G; ++h) {
        if (rot) rotate_row(q + (size_t)h * D, rot, D, q_used + (size_t)h * D);
        else memcpy(q_used + (size_t)h * D, q + (size_t)h * D, sizeof(float) * D);
    }
}

/* Importance (method section two): w_j = sigma_j^2 * sum_h q_hj^2, the query
 * energy of the group as an fp32 fma chain over ascending h, times the
 * calibration variance.  Non-positive or NaN weights become 0 (never read). */
void orc_importance(const float* q_used, const float* sigma2, int G, int D, float* w)
{
    for (int j = 0; j < D; ++j) {
        float sq = 0.0f;
        for (int h = 0; h < G; ++h) sq = fmaf(q_used[(size_t)h * D + j], q_used[(size_t)h * D + j], sq);
        float v = sigma2[j] * sq;
        w[j] = (v > 0.0f) ? v : 0.0f;
    }
}

/* Depth of one channel at water level theta (reading of the lost integer
 * solution): t = #{t in 0..3 : w > fl32(theta * 4^t)}, i.e. one more plane
 * for every factor 4 by which the weight clears the water level. */
int orc_depth_at(float w, float theta)
{
    int t = 0;
    float lvl = theta;
    for (int s = 0; s < 4; ++s) {
        if (w > lvl) ++t;
        lvl = lvl * 4.0f;
    }
    return t;
}

/* Smallest fp32 theta with fl32(theta * 4^t) >= w (w > 0): the ceiling of the
 * real quotient w / 4^t onto the fp32 grid. */
static float breakpoint(float w, int t)
{
    double d = ldexp((double)w, -2 * t);
    float f = (float)d;
    if ((double)f < d) f = nextafterf(f, INFINITY);
    return f;
}

static int cmp_float_desc(const void* a, const void* b)
{
    float x = *(const float*)a, y = *(const float*)b;
    return (x < y) - (x > y);
}

/* Water level (method section two): the smallest theta >= 0 whose depths sum
 * to at most B.  Written out as an order statistic: sum_j t_j(theta) counts
 * the pairs (j, t) whose breakpoint exceeds theta, so the level is 0 when at
 * most B pairs exist, else the (B+1)-th largest breakpoint. */
float orc_water_level(const float* w, int D, int B)
{
    float* v = (float*)malloc(sizeof(float) * 4 * (size_t)D);
    int m = 0;
    for (int j = 0; j < D; ++j)
        if (w[j] > 0.0f)
            for (int t = 0; t < 4; ++t) v[m++] = breakpoint(w[j], t);
    float theta = 0.0f;
    if (m > B) {
        qsort(v, (size_t)m, sizeof(float), cmp_float_desc);
        theta = v[B];
    }
    free(v);
    return theta;
}

typedef struct {
    float key;
    int idx;
} orc_rank_t;

static int cmp_rank(const void* a, const void* b)
{
    const orc_rank_t* x = (const orc_rank_t*)a;
    const orc_rank_t* y = (const orc_rank_t*)b;
    if (x->key > y->key) return -1;
    if (x->key < y->key) return 1;
    return (x->idx > y->idx) - (x->idx < y->idx);
}

/* Full plan for one pair.  mode WATERFILL: budget = plane bits per token.
 * mode TOPR: the fixed-depth r-channel scan (SparQ-style ranking by the
 * group's query energy sum_h q_hj^2, ties to the lower channel), budget = r,
 * every chosen channel read at 4 planes.  mode UNIFORM: every channel at
 * depth = budget (the thumbnail scan).  Returns theta (0 for fixed plans). */
float orc_plan(const float* q, const float* sigma2, const float* rot, int G, int D, int budget,
               int mode, uint8_t* depth, float* q_used)
{
    orc_query_used(q, rot, G, D, q_used);
    float theta = 0.0f;
    if (mode == ORC_PLAN_WATERFILL) {
        float* w = (float*)malloc(sizeof(float) * (size_t)D);
        orc_importance(q_used, sigma2, G, D, w);
        theta = orc_water_level(w, D, budget);
        for (int j = 0; j < D; ++j) depth[j] = (uint8_t)orc_depth_at(w[j], theta);
        free(w);
    } else if (mode == ORC_PLAN_TOPR) {
        orc_rank_t* r = (orc_rank_t*)malloc(sizeof(orc_rank_t) * (size_t)D);
        for (int j = 0; j < D; ++j) {
            float sq = 0.0f;
            for (int h = 0; h < G; ++h) sq = fmaf(q_used[(size_t)h * D + j], q_used[(size_t)h * D + j], sq);
            r[j].key = sq;
            r[j].idx = j;
        }
        qsort(r, (size_t)D, sizeof(orc_rank_t), cmp_rank);
        memset(depth, 0, (size_t)D);
        for (int i = 0; i < budget && i < D; ++i) depth[r[i].idx] = 4;
        free(r);
    } else {
        for (int j = 0; j < D; ++j) depth[j] = (uint8_t)budget;
    }
    return theta;
}

/* ------------------------------------------------------------------- scan */

/* Approximate scores, fixed-point contract.  The real value is the same dot
 * product of the query with the prefix-decoded key; it is evaluated so that
 * the sum is exact and only the final result is rounded:
 *   - sigma_h = 31 - floor(log2 max_j |q_hj|) over the read channels (0 if
 *     they are all zero), so that |q_hj| * 2^sigma_h < 2^32;
 *   - per 64-token block b, E_b = f_b - 15 with f_b the largest binary16
 *     exponent field among the read channels' scales in the block (at least
 *     1, so subnormal and zero scales count as 2^-14): every read scale is
 *     below 2^(E_b + 1);
 *   - coefficient A_hjb = trunc(fl32(fl32(q_hj * 2^sigma_h) * scale_jb) *
 *     2^-(E_b + 3)), an integer with |A| <= 2^30;
 *   - with c' = c_t * 2^(4-t) (the prefix with zeros below it) and
 *     d_j = 2^(4-t_j) - 16, the prefix key is (2 c' + d) * scale / 16, so
 *     S_i = sum_j A_hjb * (2 c'_ij + d_j) is an exact integer and the score
 *     is fl32(S_i * 2^(E_b - 1 - sigma_h)), one rounding to nearest even.
 * Padding tokens are -inf.  Bound (vs the real dot product): at most
 * 15 * (#read channels) * 2^(E_b - 1 - sigma_h) + 2^-24 * sum_j |q_hj k_ij|
 * before the final rounding. */
static int floor_log2_pos(double x) /* x > 0 */
{
    int e;
    frexp(x, &e);
    return e - 1;
}

void orc_scores(const uint64_t* planes, const uint16_t* scales, int64_t n, int D,
                const uint8_t* depth, const float* q_used, int G, float* scores)
{
    int64_t nb = (n + 63) / 64;
    int64_t npad = nb * 64;
    int64_t* A = (int64_t*)malloc(sizeof(int64_t) * (size_t)D);
    for (int h = 0; h < G; ++h) {
        const float* q = q_used + (size_t)h * D;
        float qmax = 0.0f;
        for (int j = 0; j < D; ++j)
            if (depth[j] > 0 && fabsf(q[j]) > qmax) qmax = fabsf(q[j]);
        int sigma = qmax > 0.0f ? 31 - floor_log2_pos((double)qmax) : 0;
        for (int64_t b = 0; b < nb; ++b) {
            int ef = 1; /* largest exponent field of the read scales (subnormals and 0 count as 1) */
            for (int j = 0; j < D; ++j) {
                int f = (scales[(size_t)j * nb + b] >> 10) & 31;
                if (depth[j] > 0 && f > ef) ef = f;
            }
            int E = ef - 15;
            for (int j = 0; j < D; ++j) {
                A[j] = 0;
                if (depth[j] == 0) continue;
                float qs = ldexpf(q[j], sigma);                 /* exact */
                float pr = qs * orc_f16_to_f32(scales[(size_t)j * nb + b]); /* fl32 */
                A[j] = (int64_t)truncf(ldexpf(pr, -(E + 3)));   /* exact scaling */
            }
            for (int i = 0; i < 64; ++i) {
                int64_t tok = 64 * b + i;
                if (tok >= n) {
                    scores[(size_t)h * npad + tok] = -INFINITY;
                    continue;
                }
                int64_t S = 0;
                for (int j = 0; j < D; ++j) {
                    int t = depth[j];
                    if (t == 0) continue;
                    int cp = orc_prefix_code(planes, nb, j, tok, t) << (4 - t);
                    S += A[j] * (int64_t)(2 * cp + (1 << (4 - t)) - 16);
                }
                scores[(size_t)h * npad + tok] = (float)ldexp((double)S, E - 1 - sigma);
            }
        }
    }
    free(A);
}

/* The same sum in double (the real-valued definition, for tolerances). */
void orc_scores_f64(const uint64_t* planes, const uint16_t* scales, int64_t n, int D,
                    const uint8_t* depth, const float* q_used, int G, double* scores)
{
    int64_t nb = (n + 63) / 64;
    for (int h = 0; h < G; ++h)
        for (int64_t i = 0; i < n; ++i) {
            double acc = 0.0;
            for (int j = 0; j < D; ++j) {
                int t = depth[j];
                if (t == 0) continue;
                int ct = orc_prefix_code(planes, nb, j, i, t);
                acc += (double)q_used[(size_t)h * D + j] *
                       (double)orc_dequant(ct, t, scales[(size_t)j * nb + i / 64]);
            }
            scores[(size_t)h * n + i] = acc;
        }
}

/* ------------------------------------------------------------------ top-k */

static int cmp_rank_f(const void* a, const void* b) { return cmp_rank(a, b); }

/* Top-k of one head (method: every query head keeps its k best keys):
 * order by (score descending, token index ascending); -0 and +0 are equal.
 * Only the n valid tokens take part.  Writes k indices and their scores. */
void orc_topk(const float* scores, int64_t n, int k, int32_t* idx, float* val)
{
    orc_rank_t* r = (orc_rank_t*)malloc(sizeof(orc_rank_t) * (size_t)n);
    for (int64_t i = 0; i < n; ++i) {
        r[i].key = scores[i] == 0.0f ? 0.0f : scores[i];
        r[i].idx = (int)i;
    }
    qsort(r, (size_t)n, sizeof(orc_rank_t), cmp_rank_f);
    for (int i = 0; i < k; ++i) {
        idx[i] = r[i].idx;
        if (val) val[i] = scores[r[i].idx];
    }
    free(r);
}

static int cmp_i32(const void* a, const void* b)
{
    int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return (x > y) - (x < y);
}

/* Union over the G heads of one KV head (the rows the group fetches):
 * ascending, duplicates removed, padded with -1 to G*k.  Returns its length. */
int orc_union(const int32_t* idx, int G, int k, int32_t* out)
{
    int m = G * k;
    int32_t* tmp = (int32_t*)malloc(sizeof(int32_t) * (size_t)m);
    memcpy(tmp, idx, sizeof(int32_t) * (size_t)m);
    qsort(tmp, (size_t)m, sizeof(int32_t), cmp_i32);
    int len = 0;
    for (int i = 0; i < m; ++i)
        if (len == 0 || tmp[i] != out[len - 1]) out[len++] = tmp[i];
    for (int i = len; i < m; ++i) out[i] = -1;
    free(tmp);
    return len;
}

/* One decode step for one pair as the cpu baseline times it: plan, scores,
 * top-k per head and the union.  scores: [G][nb*64] scratch. */
int orc_step(const uint64_t* planes, const uint16_t* scales, int64_t n, int D, const float* q,
             const float* sigma2, const float* rot, int G, int budget, int mode, int k,
             uint8_t* depth, float* q_used, float* scores, int32_t* topk_idx, int32_t* union_idx)
{
    int64_t npad = ((n + 63) / 64) * 64;
    orc_plan(q, sigma2, rot, G, D, budget, mode, depth, q_used);
    orc_scores(planes, scales, n, D, depth, q_used, G, scores);
    for (int h = 0; h < G; ++h)
        orc_topk(scores + (size_t)h * npad, n, k, topk_idx + (size_t)h * k, NULL);
    return orc_union(topk_idx, G, k, union_idx);
}

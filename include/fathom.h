/*
 * fathom.h -- C ABI of the Fathom per-query variable-depth key scan for
 * AMD Instinct MI355X (gfx950).
 *
 * Method: "Fathom: Per-Query Read Depth for Sparse Decoding over Offloaded KV
 * Caches" (arXiv 2609.17652), as described on the yeyulingfeng.com write-up
 * (sections "方法一" -- keys as bit planes, "方法二" -- reverse water-filling
 * per query group, "基座选择" -- raw versus rotated basis) and the bit-plane
 * figure of the paotong.dev page.  A decode step scores all n cached keys of
 * one KV head against its G query heads from a 4-bit bit-plane index, reading
 * only a per-channel prefix of planes, and keeps the k best keys per query
 * head plus their union per KV head.
 *
 * Conventions shared by every entry point
 *  - A "pair" is one (layer, KV head).  P pairs (1 <= P <= FATHOM_MAX_PAIRS)
 *    are processed per call; every array below is pair-major and densely
 *    packed.
 *  - All pointers are DEVICE pointers (hipMalloc'd, or host memory mapped
 *    into the device address space with hipHostMalloc(..., Mapped) -- the
 *    scan reads such an index over the host link), owned by the caller, and
 *    16-byte aligned.  The library never allocates or frees caller memory.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Calls only enqueue work: they do not synchronise.  Argument checks run
 *    on the host before anything is enqueued; a failed check enqueues nothing.
 *  - Return value: FATHOM_OK (0) or a negative FATHOM_ERR_* code; launch
 *    failures are reported as FATHOM_ERR_HIP.  Nothing throws.
 *  - D (channels per head) must satisfy 1 <= D <= 128; G (query heads per KV
 *    head) 1 <= G <= 8; n (tokens) >= 1.  nb = ceil(n / 64) blocks,
 *    npad = 64 * nb.  Tokens n..npad-1 of the last block are padding.
 *
 * Index layout (per pair), with rows of L blocks:
 *    planes [D][4][L] uint64 -- word (j, s, b): bit i is bit (3 - s) of the
 *                               4-bit code of token 64*b + i in channel j
 *                               (s = 0 is the sign plane).  A channel's
 *                               t-plane prefix is t*L contiguous words.
 *    scales [D][L]    uint16 -- IEEE binary16 block max |x| of (channel, block).
 *  L = nb for a dense index.  An index meant to grow is allocated with a
 *  capacity of nb_cap >= nb blocks per row (L = nb_cap) and filled or
 *  extended with fathom_pack_range; calls that read it take nb_cap.
 *  Footprint: 68 bytes per token per pair at D = 128.
 *  The scan entry points need one pair's plane rows to span less than 2^31
 *  bytes (D * 32 * L < 2^31; at D = 128, L < 524,288 blocks or 33.5M tokens
 *  per pair) and return FATHOM_ERR_UNSUPPORTED otherwise.
 */
#ifndef FATHOM_H
#define FATHOM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FATHOM_ABI_VERSION 2

#define FATHOM_OK 0
#define FATHOM_ERR_ARG (-1)         /* null pointer, bad enum, bad budget/k  */
#define FATHOM_ERR_SHAPE (-2)       /* P, n, D or G out of range             */
#define FATHOM_ERR_ALIGN (-3)       /* pointer not 16-byte aligned           */
#define FATHOM_ERR_WORKSPACE (-4)   /* workspace missing or too small        */
#define FATHOM_ERR_UNSUPPORTED (-5) /* valid but not supported (k > 4096 ...) */
#define FATHOM_ERR_HIP (-6)         /* a HIP launch or query failed          */

#define FATHOM_DTYPE_F32 0
#define FATHOM_DTYPE_BF16 1

#define FATHOM_PLAN_WATERFILL 0 /* budget = plane bits per token (0..4D)            */
#define FATHOM_PLAN_TOPR 1      /* budget = r channels read at 4 planes (0..D)      */
#define FATHOM_PLAN_UNIFORM 2   /* budget = depth of every channel (0..4)           */

#define FATHOM_MAX_K 4096
#define FATHOM_MAX_PAIRS 65535 /* P per call (pairs run on the grid's y axis) */

int fathom_abi_version(void);
const char* fathom_strerror(int status);

/*
 * fathom_pack -- quantise keys into the bit-plane index (method section one).
 *
 *   keys   [P][n][D]  token-major, float32 (dtype F32) or bfloat16 (BF16)
 *   rot    [P][D][D]  or NULL.  When given, channel j of the stored key is
 *                     sum_d rot[d][j] * key[d], evaluated as a float32 fused
 *                     multiply-add chain over ascending d (the rotated basis
 *                     of the basis-choice section).
 *   planes [P][D][4][nb], scales [P][D][nb]  outputs (layout above).
 *
 * Per (block, channel): m = max |x| over the block's valid tokens, stored as
 * binary16 round-to-nearest-even (saturated at 65504); cell width
 * delta = scale / 8; code c = clamp(floor(x / delta) + 8, 0, 15) with the
 * exact real floor; a zero scale gives code 8; padding tokens get code 8.
 * Keys must be finite.  Errors: ERR_ARG (null, bad dtype), ERR_SHAPE, ERR_ALIGN.
 */
int fathom_pack(const void* keys, int32_t dtype, int32_t P, int64_t n, int32_t D,
                const float* rot, uint64_t* planes, uint16_t* scales, void* stream);

/*
 * fathom_pack_range -- pack tokens [tok0, tok0 + m) of every pair into an
 * index with rows of nb_cap blocks, leaving all other blocks untouched.
 * Each block is quantised on its own (its scale is its own block max), so
 * packing a range gives bit for bit the words and scales that fathom_pack
 * of the whole sequence gives for those blocks.  Appending to a decode
 * cache: when token n-1 arrives, pack the raw keys of its block (tokens
 * 64*floor((n-1)/64) .. n-1, held by the caller's KV cache) with
 * tok0 = 64*floor((n-1)/64); the block's scale is recomputed from all of
 * them.  The pages do not describe appends; this is the plainest reading of
 * their per-block quantiser.
 *
 *   keys   [P][m][D]  the keys of the range, as in fathom_pack
 *   tok0   first token, a multiple of 64
 *   m      tokens in the range, 1 <= m, tok0 + m <= 64 * nb_cap
 *   rot, planes, scales  as in fathom_pack, rows of nb_cap blocks
 * Tokens of the last block beyond the range are padding (code 8).
 * Errors: ERR_ARG (null, dtype, tok0 not a multiple of 64), ERR_SHAPE,
 * ERR_ALIGN.
 */
int fathom_pack_range(const void* keys, int32_t dtype, int32_t P, int64_t tok0, int64_t m,
                      int32_t D, const float* rot, uint64_t* planes, uint16_t* scales,
                      int64_t nb_cap, void* stream);

/*
 * fathom_plan -- per-pair read plan (method section two; basis section).
 *
 *   q       [P][G][D] float32 query heads of each KV-head group
 *   sigma2  [P][D]    float32 calibration variance of each stored coordinate
 *                     (rotated-coordinate variances when keys are rotated)
 *   rot     [P][D][D] or NULL: when given, q_used = rot^T q per head, each
 *                     output a float32 fma chain over ascending d
 *   budget, mode      see FATHOM_PLAN_*
 * Outputs:
 *   depth    [P][D] uint8   planes read per channel, 0..4
 *   active   [P][D] int16   channels with depth > 0, ascending; rest -1
 *   n_active [P]    int32
 *   theta    [P]    float32 water level (0 for the fixed plans)
 *   q_used   [P][G][D] float32 query actually scored (q, or rot^T q)
 *
 * WATERFILL: w_j = sigma2_j * sum_h q_used_hj^2 (float32 fma chain over
 * ascending h, then one product; non-positive weights are 0);
 * t_j(theta) = #{t in 0..3 : w_j > theta * 4^t}; theta = the smallest
 * non-negative float32 with sum_j t_j(theta) <= budget (exact search over the
 * float32 bit patterns).  TOPR: the `budget` channels of largest
 * sum_h q_used_hj^2 (ties to the lower channel) get depth 4.  UNIFORM: every
 * channel gets depth `budget`.
 * Errors: ERR_ARG (null, bad mode, budget out of range), ERR_SHAPE, ERR_ALIGN.
 */
int fathom_plan(const float* q, const float* sigma2, const float* rot, int32_t P, int32_t G,
                int32_t D, int32_t budget, int32_t mode, uint8_t* depth, int16_t* active,
                int32_t* n_active, float* theta, float* q_used, void* stream);

/*
 * fathom_scan -- approximate scores of every key (method section two: read
 * the t_j-plane prefix of each active channel; limitations section: one
 * shift-and-mask per extracted bit and G multiply-adds per element).
 *
 *   planes, scales       the index (may be host-mapped memory)
 *   nb_cap               blocks per index row: 0 for a dense index (nb),
 *                        else the capacity it was allocated with (>= nb)
 *   depth, active, n_active, q_used   a plan from fathom_plan
 *   scores [P][G][npad]  float32 output: the dot product of q_used[h]
 *       with the dequantised prefix keys, khat_ij = (2 c_t + 1 - 2^t) *
 *       2^-t * scale (c_t = c >> (4 - t_j)), evaluated exactly and rounded
 *       once.  Fixed-point contract, per head h and 64-token block b:
 *         sigma_h = 31 - floor(log2 max_j |q_used[h][j]|) over the read
 *                   channels (0 if all are 0);
 *         E_b     = f_b - 15, f_b the largest binary16 exponent field of the
 *                   read channels' scales in the block (at least 1);
 *         A_hjb   = trunc(fl32(fl32(q_used[h][j] 2^sigma_h) * scale_jb) *
 *                   2^-(E_b + 3)), an integer with |A| <= 2^30;
 *         S_i     = sum_j A_hjb (2 c'_ij + 2^(4-t_j) - 16), c' = c_t 2^(4-t_j),
 *                   an exact integer;
 *         score   = fl32(S_i 2^(E_b - 1 - sigma_h)), round to nearest even.
 *       The result differs from the real dot product by at most
 *       15 (#read channels) 2^(E_b - 1 - sigma_h) + 2^-24 sum_j |q k| before
 *       the final rounding.  Padding tokens are -inf.
 * Errors: ERR_ARG (null), ERR_SHAPE, ERR_ALIGN, ERR_UNSUPPORTED (a pair's
 * plane rows span 2^31 bytes or more).
 */
int fathom_scan(const uint64_t* planes, const uint16_t* scales, int32_t P, int32_t D, int64_t n,
                int64_t nb_cap, const uint8_t* depth, const int16_t* active,
                const int32_t* n_active, const float* q_used, int32_t G, float* scores,
                void* stream);

/*
 * fathom_topk -- the k best keys of every query head and their union per KV
 * head (the winner rows a step fetches).  The byte-accounting section of the
 * yeyulingfeng.com write-up ("先算一笔字节账") defines the selection: each
 * query head keeps its k = 512 highest-scoring keys, and the G heads of a KV
 * head fetch the union of their winners, at most G * k rows; its opening
 * paragraph fixes that every key is scored before any is chosen.  Ties in
 * score go to the lower token index and the union is listed in ascending
 * order; the pages leave both open.
 *
 *   scores    [P][G][npad] from fathom_scan
 *   topk_idx  [P][G][k] int32 token indices ordered by (score descending,
 *             index ascending); -0 and +0 compare equal; padding excluded
 *   topk_val  [P][G][k] float32 their scores, or NULL
 *   union_idx [P][G*k] int32 ascending union of the G lists, padded with -1
 *   union_len [P] int32
 *   ws        device workspace of at least fathom_topk_workspace_bytes()
 * Requires 1 <= k <= min(n, FATHOM_MAX_K).  Errors: ERR_ARG, ERR_SHAPE,
 * ERR_ALIGN, ERR_UNSUPPORTED (k > 4096), ERR_WORKSPACE.
 */
size_t fathom_topk_workspace_bytes(int32_t P, int32_t G, int64_t n, int32_t k);
int fathom_topk(const float* scores, int32_t P, int32_t G, int64_t n, int32_t k,
                int32_t* topk_idx, float* topk_val, int32_t* union_idx, int32_t* union_len,
                void* ws, size_t ws_bytes, void* stream);

/*
 * fathom_scan_topk -- fathom_scan followed by fathom_topk in one call,
 * without materialising the scores (the decode-step hot path).
 *
 * Same inputs as fathom_scan plus k, and the outputs of fathom_topk, which
 * are identical to fathom_scan + fathom_topk on the same inputs.  Internally:
 * the scores of one run of 32 blocks in every s runs (s ~ sqrt(n / 4k), a
 * power of two) are computed first -- as maxima of groups of 16 tokens once
 * the sample is large -- and the ceil(2k / s)-th largest sample value is
 * taken as each head's threshold (with s = 1: the exact k-th largest); one
 * pass over the whole index then keeps the scores at or above it as
 * candidates, and the k best candidates are selected exactly.  A head that
 * ends up with fewer than k candidates (the sample misjudged it) or more
 * than their capacity (massive ties) has its pair rescanned into a full
 * score row inside the workspace and is selected from there; results are
 * exact either way.  The rows are min(P, 16) pairs' worth (G * npad floats
 * each): the first failed pairs are rescanned into them by many workgroups
 * at once, and any further ones by one workgroup per row in turn, so the
 * workspace does not grow with the number of failures (at 1M tokens x 288
 * pairs, G = 4, k = 512 it is about 0.9 GB).
 *
 * An index in host memory (hipHostMalloc'd and mapped, read over the host
 * link; the call asks the HIP runtime what kind of memory `planes` is) is
 * read once per call instead of the sampled runs twice: the sample stage
 * keeps every score it computes in the workspace, and the filter pass skips
 * the sampled runs and keeps their stored scores that reach the threshold
 * instead.  This needs the larger of the two workspace layouts, which
 * fathom_scan_topk_workspace_bytes() always returns; a smaller workspace
 * that fits the device layout gives the same results without the staging.
 *   ws  device workspace of at least fathom_scan_topk_workspace_bytes().
 * Errors: as fathom_scan and fathom_topk.
 */
size_t fathom_scan_topk_workspace_bytes(int32_t P, int32_t G, int64_t n, int32_t k);
int fathom_scan_topk(const uint64_t* planes, const uint16_t* scales, int32_t P, int32_t D, int64_t n,
                     int64_t nb_cap, const uint8_t* depth, const int16_t* active,
                     const int32_t* n_active, const float* q_used, int32_t G, int32_t k,
                     int32_t* topk_idx, float* topk_val, int32_t* union_idx, int32_t* union_len,
                     void* ws, size_t ws_bytes, void* stream);

/*
 * fathom_scan_topk_stage -- the three stages of fathom_scan_topk as separate
 * calls, so that a caller can time or interleave them.  Enqueueing stages 1,
 * 2 and 3 in that order on one stream with the same arguments and workspace
 * is exactly fathom_scan_topk.
 *   stage 1: sample scores and per-head thresholds (written into ws)
 *   stage 2: the scan over every block with the threshold filter -- one
 *            kernel launch, the step's dominant kernel (for an index in
 *            host memory: over every block outside the sample, then a
 *            second launch filters the sample's stored scores)
 *   stage 3: overflow repair, exact selection and union (the outputs; they
 *            may be NULL in stages 1 and 2)
 * Errors: ERR_ARG for a stage outside 1..3, else as fathom_scan_topk.
 */
int fathom_scan_topk_stage(int32_t stage, const uint64_t* planes, const uint16_t* scales, int32_t P,
                           int32_t D, int64_t n, int64_t nb_cap, const uint8_t* depth,
                           const int16_t* active, const int32_t* n_active, const float* q_used,
                           int32_t G, int32_t k, int32_t* topk_idx, float* topk_val,
                           int32_t* union_idx, int32_t* union_len, void* ws, size_t ws_bytes,
                           void* stream);

/*
 * fathom_scan_topk_noalloc -- fathom_scan_topk for callers that cannot
 * allocate device memory: code under HIP graph capture, serving loops that
 * must not call the allocator, harnesses that forbid it.  Same arguments and
 * results as fathom_scan_topk, without ws / ws_bytes: the workspace is a
 * fixed 128 MiB scratch array inside the library, one per GPU, which this
 * call neither allocates nor frees (the first call on a device looks up that
 * device's copy).
 *
 * Limit: the call must fit the scratch with at least one repair row, i.e.
 * fathom_scan_topk_workspace_bytes computed with one row instead of
 * min(P, 16) must be at most 128 MiB (at G = 4, k = 512: 8 pairs x 4M
 * tokens, 16 x 2M or 32 x 1M fit, a layer's 8 KV heads at any context up to
 * 4M; 288 pairs x 1M do not).  Fewer rows than min(P, 16) only slow the rare
 * repair.  Larger calls return ERR_WORKSPACE before any work is enqueued.
 *
 * Every call on a GPU uses that GPU's one scratch array, whose contents are
 * left over from the last call (nothing in it needs to start at zero): calls
 * that overlap on one GPU -- on different streams, or from different host
 * threads -- race and must be serialised by the caller.  The current device
 * must be the one the pointers and the stream belong to.
 * Errors: as fathom_scan_topk, with ERR_WORKSPACE for a call too large for
 * the scratch and ERR_HIP if the scratch cannot be located.
 */
int fathom_scan_topk_noalloc(const uint64_t* planes, const uint16_t* scales, int32_t P, int32_t D,
                             int64_t n, int64_t nb_cap, const uint8_t* depth, const int16_t* active,
                             const int32_t* n_active, const float* q_used, int32_t G, int32_t k,
                             int32_t* topk_idx, float* topk_val, int32_t* union_idx, int32_t* union_len,
                             void* stream);

/*
 * fathom_gather_rows -- the winner-row fetch that follows the selection:
 * copy the union rows of every pair (the keys and values a decode step
 * attends to, at most G*k rows per KV head) out of a row table that may live
 * in mapped host memory (byte-accounting and experiments sections).
 *
 *   table      row-major table of table_rows rows of row_bytes bytes per pair
 *              (e.g. K and V of one token side by side: 2 * D * 2 bytes in
 *              bf16); pair p's token i is row p * pair_stride_rows + i, so
 *              pair_stride_rows = table_rows gives one table per pair and 0
 *              one table shared by all pairs
 *   union_idx  [P][cap] int32 ascending token indices (fathom_topk's union)
 *   union_len  [P]      int32 rows to fetch per pair (<= cap)
 *   out        [P][cap][row_bytes] device memory; rows r >= union_len[p] and
 *              indices outside [0, table_rows) are left untouched
 * row_bytes must be a positive multiple of 16 and 1 <= P <= FATHOM_MAX_PAIRS.  All
 * pointers 16-byte aligned.  Errors: ERR_ARG (null), ERR_SHAPE, ERR_ALIGN.
 */
int fathom_gather_rows(const void* table, int64_t table_rows, int64_t row_bytes,
                       int64_t pair_stride_rows, int32_t P, const int32_t* union_idx,
                       const int32_t* union_len, int32_t cap, void* out, void* stream);

/*
 * fathom_calib_covariance -- calibration statistics of each pair on the
 * device: the water-filling weights are the variances of the stored
 * coordinates, and the rotated storage is the eigenbasis of the key
 * covariance (reverse water-filling and basis-choice sections).  The
 * calibration-domain passage computes them from the session's own prefill
 * keys, one covariance per KV head.
 *
 *   keys  [P][m][D]  float32 (F32) or bfloat16 (BF16), m >= 1
 *   cov   [P][D][D]  float64 centred population covariance
 *                    sum_t (x_t - mu)(x_t - mu)^T / m, or NULL
 *   var   [P][D]     float32 channel variances (cov's diagonal rounded once),
 *                    or NULL; at least one of cov and var must be given
 *   ws    device workspace of fathom_calib_workspace_bytes(P, m, D) bytes
 * Accumulation is float64 in a fixed order (deterministic).  Errors:
 * ERR_ARG, ERR_SHAPE, ERR_WORKSPACE, ERR_ALIGN.
 */
size_t fathom_calib_workspace_bytes(int32_t P, int64_t m, int32_t D);
int fathom_calib_covariance(const void* keys, int32_t dtype, int32_t P, int64_t m, int32_t D,
                            double* cov, float* var, void* ws, size_t ws_bytes, void* stream);

/*
 * fathom_calib_basis -- eigen-decomposition of each pair's covariance by
 * cyclic Jacobi rotations (float64 matrix, float32 eigenvectors), one
 * workgroup per pair.
 *
 *   cov  [P][D][D] float64 symmetric (from fathom_calib_covariance)
 *   U    [P][D][D] float32: column c is the eigenvector of the c-th largest
 *                  eigenvalue, signed so that its largest-magnitude component
 *                  is positive -- the rot argument of fathom_pack/plan
 *   lam  [P][D]    float32 eigenvalues in descending order, clamped at 0: the
 *                  variances of the rotated coordinates (sigma2 of fathom_plan)
 * Sweeps stop when the off-diagonal norm falls below 1e-12 of the diagonal
 * norm (at most 20).  Errors: ERR_ARG, ERR_SHAPE, ERR_ALIGN.
 */
int fathom_calib_basis(const double* cov, int32_t P, int32_t D, float* U, float* lam, void* stream);

/*
 * fathom_read_probe -- measurement utility, not a step of the method: reads
 * `bytes` (rounded down to a multiple of 16) from `src` once with 16-byte
 * coalesced loads and folds them into sink[0..1023] (caller-owned device
 * memory, XOR-accumulated).  Timing it gives the read bandwidth the scan can
 * reach on that memory: HBM, or the host link for a hipHostMalloc'd mapped
 * buffer.  Errors: ERR_ARG (null, bytes < 16), ERR_ALIGN.
 */
int fathom_read_probe(const void* src, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FATHOM_H */

// C ABI entry points (declared in include/fathom.h): argument checks on the
// host, then asynchronous launches on the caller's stream.
#include <mutex>

#include "../../include/fathom.h"
#include "common.h"

using namespace fathom;

namespace {

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

inline int hip_status(hipError_t e) { return e == hipSuccess ? FATHOM_OK : FATHOM_ERR_HIP; }

constexpr int64_t kMaxTokens = ((int64_t)1 << 31) - 64;  // token index fits int32
constexpr int64_t kMaxRowBlocks = (int64_t)1 << 25;      // 64 * this = 2^31 tokens

inline int check_shape(int32_t P, int64_t n, int32_t D)
{
    if (P < 1 || P > kMaxPairs || n < 1 || D < 1 || D > kMaxD) return FATHOM_ERR_SHAPE;
    if (n > kMaxTokens) return FATHOM_ERR_SHAPE;
    return FATHOM_OK;
}

// The scan kernels address a pair's planes and scales with 32-bit buffer
// offsets whose bit 31 marks a load as out of range, so a pair's plane rows
// (D channels x 4 planes x L blocks x 8 bytes) must span less than 2^31 bytes:
// at D = 128 that is L < 524,288 blocks, 33.5M tokens per pair.
inline bool scan_offsets_fit(int32_t D, int64_t ldb)
{
    return (int64_t)D * 4 * ldb * 8 < ((int64_t)1 << 31);
}

// Row stride of the index in blocks: 0 selects ceil(n / 64); anything else
// must hold the n tokens.  Returns -1 when invalid.
inline int64_t row_blocks(int64_t n, int64_t nb_cap)
{
    const int64_t nb = (n + 63) / 64;
    if (nb_cap == 0) return nb;
    if (nb_cap < nb || nb_cap > kMaxRowBlocks) return -1;
    return nb_cap;
}

// ---- the fixed scratch of fathom_scan_topk_noalloc.  Each GPU the library
// runs on holds its own copy of this array until the process ends; host
// code reaches it only through the device address hipGetSymbolAddress gives
// for the current device (the array's name on the host is not that address).
constexpr size_t kScratchBytes = (size_t)128 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];  // per device ordinal, set on the first call there

int scratch_address(void** out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return FATHOM_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return FATHOM_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return FATHOM_ERR_HIP;
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return FATHOM_OK;
}

}  // namespace

extern "C" {

int fathom_abi_version(void) { return FATHOM_ABI_VERSION; }

const char* fathom_strerror(int status)
{
    switch (status) {
    case FATHOM_OK: return "ok";
    case FATHOM_ERR_ARG: return "invalid argument";
    case FATHOM_ERR_SHAPE: return "shape out of range";
    case FATHOM_ERR_ALIGN: return "pointer not 16-byte aligned";
    case FATHOM_ERR_WORKSPACE: return "workspace missing or too small";
    case FATHOM_ERR_UNSUPPORTED: return "unsupported configuration";
    case FATHOM_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
    }
}

int fathom_pack(const void* keys, int32_t dtype, int32_t P, int64_t n, int32_t D,
                const float* rot, uint64_t* planes, uint16_t* scales, void* stream)
{
    if (!keys || !planes || !scales) return FATHOM_ERR_ARG;
    if (dtype != FATHOM_DTYPE_F32 && dtype != FATHOM_DTYPE_BF16) return FATHOM_ERR_ARG;
    int s = check_shape(P, n, D);
    if (s) return s;
    if (!aligned16(keys) || !aligned16(planes) || !aligned16(scales) || (rot && !aligned16(rot)))
        return FATHOM_ERR_ALIGN;
    return hip_status(
        launch_pack(keys, dtype, P, 0, n, D, rot, planes, scales, (n + 63) / 64, (hipStream_t)stream));
}

int fathom_pack_range(const void* keys, int32_t dtype, int32_t P, int64_t tok0, int64_t m,
                      int32_t D, const float* rot, uint64_t* planes, uint16_t* scales,
                      int64_t nb_cap, void* stream)
{
    if (!keys || !planes || !scales) return FATHOM_ERR_ARG;
    if (dtype != FATHOM_DTYPE_F32 && dtype != FATHOM_DTYPE_BF16) return FATHOM_ERR_ARG;
    int s = check_shape(P, m, D);
    if (s) return s;
    if (tok0 < 0 || tok0 % 64 != 0) return FATHOM_ERR_ARG;
    if (nb_cap < 1 || nb_cap > kMaxRowBlocks || tok0 + m > 64 * nb_cap) return FATHOM_ERR_SHAPE;
    if (!aligned16(keys) || !aligned16(planes) || !aligned16(scales) || (rot && !aligned16(rot)))
        return FATHOM_ERR_ALIGN;
    return hip_status(
        launch_pack(keys, dtype, P, tok0, m, D, rot, planes, scales, nb_cap, (hipStream_t)stream));
}

int fathom_plan(const float* q, const float* sigma2, const float* rot, int32_t P, int32_t G,
                int32_t D, int32_t budget, int32_t mode, uint8_t* depth, int16_t* active,
                int32_t* n_active, float* theta, float* q_used, void* stream)
{
    if (!q || !sigma2 || !depth || !active || !n_active || !theta || !q_used) return FATHOM_ERR_ARG;
    if (P < 1 || D < 1 || D > kMaxD || G < 1 || G > kMaxG) return FATHOM_ERR_SHAPE;
    if (mode == FATHOM_PLAN_WATERFILL) {
        if (budget < 0 || budget > 4 * D) return FATHOM_ERR_ARG;
    } else if (mode == FATHOM_PLAN_TOPR) {
        if (budget < 0 || budget > D) return FATHOM_ERR_ARG;
    } else if (mode == FATHOM_PLAN_UNIFORM) {
        if (budget < 0 || budget > 4) return FATHOM_ERR_ARG;
    } else {
        return FATHOM_ERR_ARG;
    }
    const void* ps[] = {q, sigma2, depth, active, n_active, theta, q_used};
    for (const void* p : ps)
        if (!aligned16(p)) return FATHOM_ERR_ALIGN;
    if (rot && !aligned16(rot)) return FATHOM_ERR_ALIGN;
    return hip_status(launch_plan(q, sigma2, rot, P, G, D, budget, mode, depth, active, n_active,
                                  theta, q_used, (hipStream_t)stream));
}

int fathom_scan(const uint64_t* planes, const uint16_t* scales, int32_t P, int32_t D, int64_t n,
                int64_t nb_cap, const uint8_t* depth, const int16_t* active,
                const int32_t* n_active, const float* q_used, int32_t G, float* scores,
                void* stream)
{
    if (!planes || !scales || !depth || !active || !n_active || !q_used || !scores)
        return FATHOM_ERR_ARG;
    int s = check_shape(P, n, D);
    if (s) return s;
    const int64_t ldb = row_blocks(n, nb_cap);
    if (ldb < 0) return FATHOM_ERR_SHAPE;
    if (G < 1 || G > kMaxG) return FATHOM_ERR_SHAPE;
    if (!scan_offsets_fit(D, ldb)) return FATHOM_ERR_UNSUPPORTED;
    const void* ps[] = {planes, scales, depth, active, n_active, q_used, scores};
    for (const void* p : ps)
        if (!aligned16(p)) return FATHOM_ERR_ALIGN;
    return hip_status(launch_scan(planes, scales, P, D, n, ldb, depth, active, n_active, q_used, G,
                                  scores, (hipStream_t)stream));
}

size_t fathom_topk_workspace_bytes(int32_t P, int32_t G, int64_t n, int32_t k)
{
    if (P < 1 || G < 1 || G > kMaxG || n < 1 || k < 1 || k > n || k > kMaxK) return 0;
    return topk_layout(P, G, n, k).bytes;
}

int fathom_topk(const float* scores, int32_t P, int32_t G, int64_t n, int32_t k,
                int32_t* topk_idx, float* topk_val, int32_t* union_idx, int32_t* union_len,
                void* ws, size_t ws_bytes, void* stream)
{
    if (!scores || !topk_idx || !union_idx || !union_len) return FATHOM_ERR_ARG;
    if (P < 1 || G < 1 || G > kMaxG || n < 1) return FATHOM_ERR_SHAPE;
    if (n > ((int64_t)1 << 31) - 64) return FATHOM_ERR_SHAPE;
    if (k < 1 || k > n) return FATHOM_ERR_ARG;
    if (k > kMaxK || G * k > kMaxUnion) return FATHOM_ERR_UNSUPPORTED;
    const void* ps[] = {scores, topk_idx, union_idx, union_len};
    for (const void* p : ps)
        if (!aligned16(p)) return FATHOM_ERR_ALIGN;
    if (topk_val && !aligned16(topk_val)) return FATHOM_ERR_ALIGN;
    const TopkLayout L = topk_layout(P, G, n, k);
    if (!ws || ws_bytes < L.bytes) return FATHOM_ERR_WORKSPACE;
    if (!aligned16(ws)) return FATHOM_ERR_ALIGN;
    return hip_status(launch_topk(scores, P, G, n, k, topk_idx, topk_val, union_idx, union_len, ws, L,
                                  (hipStream_t)stream));
}

size_t fathom_scan_topk_workspace_bytes(int32_t P, int32_t G, int64_t n, int32_t k)
{
    if (P < 1 || G < 1 || G > kMaxG || n < 1 || k < 1 || k > n || k > kMaxK) return 0;
    // enough for either layout: an index in device memory, or one read over the host link
    const size_t dev = topk_layout(P, G, n, k).bytes_fused;
    const size_t host = topk_layout(P, G, n, k, kRepairSlots, true).bytes_fused;
    return dev > host ? dev : host;
}

// Whether the scan reads this index over the host link (memory the HIP
// runtime knows as host memory, e.g. hipHostMalloc'd and mapped).  An
// address the runtime does not know is taken as device memory, and the
// error that query leaves is cleared so that a later launch check does not
// report it.
static bool host_resident(const void* p)
{
    hipPointerAttribute_t at{};
    if (hipPointerGetAttributes(&at, p) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    return at.type == hipMemoryTypeHost;
}

// Argument checks shared by the fused entry points; fills the scan's
// arguments.  Returns FATHOM_OK or the error.
static int scan_topk_check(const uint64_t* planes, const uint16_t* scales, int32_t P, int32_t D,
                           int64_t n, int64_t nb_cap, const uint8_t* depth, const int16_t* active,
                           const int32_t* n_active, const float* q_used, int32_t G, int32_t k,
                           int32_t* topk_idx, float* topk_val, int32_t* union_idx, int32_t* union_len,
                           int stages, ScanArgs& a)
{
    if (!planes || !scales || !depth || !active || !n_active || !q_used) return FATHOM_ERR_ARG;
    if ((stages & 4) && (!topk_idx || !union_idx || !union_len)) return FATHOM_ERR_ARG;
    int s = check_shape(P, n, D);
    if (s) return s;
    const int64_t ldb = row_blocks(n, nb_cap);
    if (ldb < 0) return FATHOM_ERR_SHAPE;
    if (G < 1 || G > kMaxG) return FATHOM_ERR_SHAPE;
    if (!scan_offsets_fit(D, ldb)) return FATHOM_ERR_UNSUPPORTED;
    if (k < 1 || k > n) return FATHOM_ERR_ARG;
    if (k > kMaxK || G * k > kMaxUnion) return FATHOM_ERR_UNSUPPORTED;
    const void* ps[] = {planes, scales, depth, active, n_active, q_used};
    for (const void* p : ps)
        if (!aligned16(p)) return FATHOM_ERR_ALIGN;
    if (stages & 4) {
        const void* os[] = {topk_idx, union_idx, union_len};
        for (const void* p : os)
            if (!aligned16(p)) return FATHOM_ERR_ALIGN;
        if (topk_val && !aligned16(topk_val)) return FATHOM_ERR_ALIGN;
    }
    a = ScanArgs{};
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
    return FATHOM_OK;
}

static int scan_topk_impl(const uint64_t* planes, const uint16_t* scales, int32_t P, int32_t D,
                          int64_t n, int64_t nb_cap, const uint8_t* depth, const int16_t* active,
                          const int32_t* n_active, const float* q_used, int32_t G, int32_t k,
                          int32_t* topk_idx, float* topk_val, int32_t* union_idx,
                          int32_t* union_len, void* ws, size_t ws_bytes, void* stream, int stages)
{
    ScanArgs a;
    const int s = scan_topk_check(planes, scales, P, D, n, nb_cap, depth, active, n_active, q_used, G, k,
                                  topk_idx, topk_val, union_idx, union_len, stages, a);
    if (s) return s;
    // over the host link, the sample's scores are kept for stage 2 when the
    // workspace holds them (the results are the same either way)
    TopkLayout L = topk_layout(P, G, n, k);
    if (host_resident(planes)) {
        const TopkLayout Ls = topk_layout(P, G, n, k, kRepairSlots, true);
        if (ws && ws_bytes >= Ls.bytes_fused) L = Ls;
    }
    if (!ws || ws_bytes < L.bytes_fused) return FATHOM_ERR_WORKSPACE;
    if (!aligned16(ws)) return FATHOM_ERR_ALIGN;
    return hip_status(launch_scan_topk(a, P, G, k, topk_idx, topk_val, union_idx, union_len, ws, L,
                                       stages, (hipStream_t)stream));
}

int fathom_scan_topk(const uint64_t* planes, const uint16_t* scales, int32_t P, int32_t D, int64_t n,
                     int64_t nb_cap, const uint8_t* depth, const int16_t* active,
                     const int32_t* n_active, const float* q_used, int32_t G, int32_t k,
                     int32_t* topk_idx, float* topk_val, int32_t* union_idx, int32_t* union_len,
                     void* ws, size_t ws_bytes, void* stream)
{
    return scan_topk_impl(planes, scales, P, D, n, nb_cap, depth, active, n_active, q_used, G, k,
                          topk_idx, topk_val, union_idx, union_len, ws, ws_bytes, stream, 7);
}

int fathom_scan_topk_stage(int32_t stage, const uint64_t* planes, const uint16_t* scales, int32_t P,
                           int32_t D, int64_t n, int64_t nb_cap, const uint8_t* depth,
                           const int16_t* active, const int32_t* n_active, const float* q_used,
                           int32_t G, int32_t k, int32_t* topk_idx, float* topk_val,
                           int32_t* union_idx, int32_t* union_len, void* ws, size_t ws_bytes,
                           void* stream)
{
    if (stage < 1 || stage > 3) return FATHOM_ERR_ARG;
    return scan_topk_impl(planes, scales, P, D, n, nb_cap, depth, active, n_active, q_used, G, k,
                          topk_idx, topk_val, union_idx, union_len, ws, ws_bytes, stream,
                          1 << (stage - 1));
}

int fathom_scan_topk_noalloc(const uint64_t* planes, const uint16_t* scales, int32_t P, int32_t D,
                             int64_t n, int64_t nb_cap, const uint8_t* depth, const int16_t* active,
                             const int32_t* n_active, const float* q_used, int32_t G, int32_t k,
                             int32_t* topk_idx, float* topk_val, int32_t* union_idx, int32_t* union_len,
                             void* stream)
{
    ScanArgs a;
    int s = scan_topk_check(planes, scales, P, D, n, nb_cap, depth, active, n_active, q_used, G, k,
                            topk_idx, topk_val, union_idx, union_len, 7, a);
    if (s) return s;
    // as many repair rows as the scratch holds, at least one (the results do
    // not depend on the count: the rows only bound the repair's parallelism)
    int rows = P < kRepairSlots ? P : kRepairSlots;
    TopkLayout L = topk_layout(P, G, n, k, rows);
    while (L.bytes_fused > kScratchBytes && rows > 1) L = topk_layout(P, G, n, k, --rows);
    if (L.bytes_fused > kScratchBytes) return FATHOM_ERR_WORKSPACE;
    if (host_resident(planes)) {  // the staged sample, where the scratch holds it
        const TopkLayout Ls = topk_layout(P, G, n, k, rows, true);
        if (Ls.bytes_fused <= kScratchBytes) L = Ls;
    }
    void* ws = nullptr;
    if ((s = scratch_address(&ws)) != FATHOM_OK) return s;
    return hip_status(launch_scan_topk(a, P, G, k, topk_idx, topk_val, union_idx, union_len, ws, L, 7,
                                       (hipStream_t)stream));
}

int fathom_gather_rows(const void* table, int64_t table_rows, int64_t row_bytes,
                       int64_t pair_stride_rows, int32_t P, const int32_t* union_idx,
                       const int32_t* union_len, int32_t cap, void* out, void* stream)
{
    if (!table || !union_idx || !union_len || !out) return FATHOM_ERR_ARG;
    if (P < 1 || cap < 1 || table_rows < 1 || row_bytes < 16 || row_bytes % 16 != 0 ||
        pair_stride_rows < 0)
        return FATHOM_ERR_SHAPE;
    if (pair_stride_rows != 0 && pair_stride_rows < table_rows) return FATHOM_ERR_SHAPE;
    // pairs run on grid.y; the pieces of one pair's rows on grid.x
    if (P > kMaxPairs || (int64_t)cap * (row_bytes / 16) > ((int64_t)1 << 40)) return FATHOM_ERR_SHAPE;
    const void* ps[] = {table, union_idx, union_len, out};
    for (const void* p : ps)
        if (!aligned16(p)) return FATHOM_ERR_ALIGN;
    return hip_status(launch_gather(table, table_rows, row_bytes, pair_stride_rows, P, union_idx,
                                    union_len, cap, out, (hipStream_t)stream));
}

size_t fathom_calib_workspace_bytes(int32_t P, int64_t m, int32_t D)
{
    if (P < 1 || P > kMaxPairs || m < 1 || m > kMaxTokens || D < 1 || D > kMaxD) return 0;
    return calib_workspace_bytes(P, m, D);
}

int fathom_calib_covariance(const void* keys, int32_t dtype, int32_t P, int64_t m, int32_t D,
                            double* cov, float* var, void* ws, size_t ws_bytes, void* stream)
{
    if (!keys || (!cov && !var)) return FATHOM_ERR_ARG;
    if (dtype != FATHOM_DTYPE_F32 && dtype != FATHOM_DTYPE_BF16) return FATHOM_ERR_ARG;
    int s = check_shape(P, m, D);
    if (s) return s;
    if (!ws || ws_bytes < calib_workspace_bytes(P, m, D)) return FATHOM_ERR_WORKSPACE;
    if (!aligned16(keys) || !aligned16(ws) || (cov && !aligned16(cov)) || (var && !aligned16(var)))
        return FATHOM_ERR_ALIGN;
    return hip_status(launch_calib_covariance(keys, dtype, P, m, D, cov, var, ws, (hipStream_t)stream));
}

int fathom_calib_basis(const double* cov, int32_t P, int32_t D, float* U, float* lam, void* stream)
{
    if (!cov || !U || !lam) return FATHOM_ERR_ARG;
    if (P < 1 || P > kMaxPairs || D < 1 || D > kMaxD) return FATHOM_ERR_SHAPE;
    if (!aligned16(cov) || !aligned16(U) || !aligned16(lam)) return FATHOM_ERR_ALIGN;
    return hip_status(launch_calib_basis(cov, P, D, U, lam, (hipStream_t)stream));
}

int fathom_read_probe(const void* src, size_t bytes, uint32_t* sink, void* stream)
{
    if (!src || !sink || bytes < 16) return FATHOM_ERR_ARG;
    if (!aligned16(src) || !aligned16(sink)) return FATHOM_ERR_ALIGN;
    return hip_status(launch_read_probe(src, bytes, sink, (hipStream_t)stream));
}

}  // extern "C"

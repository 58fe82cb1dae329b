// Winner-row fetch: after the top-k, a decode step reads the union rows of
// every KV head (the yeyulingfeng.com write-up of Fathom, byte-accounting
// section: at most G*k rows per KV head, about 200 MB per step, flat in n;
// experiments section: in the offloaded setting these rows cross the host
// link together with the scan).
//
// Each lane moves 16-byte pieces; the 16 (or more) lanes of one row read it
// contiguously, and every lane keeps kPieces independent loads in flight so
// that a link with microsecond latency stays busy.
#include "common.h"

namespace fathom {
namespace {

constexpr int kPieces = 4;

__global__ __launch_bounds__(256) void gather_kernel(const uint4* __restrict__ table,
                                                     int64_t table_rows, int64_t pair_stride,
                                                     int64_t pieces_per_row,
                                                     const int32_t* __restrict__ idx,
                                                     const int32_t* __restrict__ len, int cap,
                                                     uint4* __restrict__ out)
{
    const int p = blockIdx.y;
    const int64_t rows = len[p] < cap ? len[p] : cap;
    const int64_t total = rows * pieces_per_row;
    const int64_t base = ((int64_t)blockIdx.x * 256 * kPieces) + threadIdx.x;
    uint4 v[kPieces];
    int64_t dst[kPieces];
#pragma unroll
    for (int u = 0; u < kPieces; ++u) {
        const int64_t c = base + (int64_t)u * 256;
        dst[u] = -1;
        if (c < total) {
            const int64_t r = c / pieces_per_row, part = c - r * pieces_per_row;
            const int64_t tok = idx[(size_t)p * cap + r];
            if (tok >= 0 && tok < table_rows) {
                v[u] = table[((size_t)p * pair_stride + tok) * pieces_per_row + part];
                dst[u] = ((int64_t)p * cap + r) * pieces_per_row + part;
            }
        }
    }
#pragma unroll
    for (int u = 0; u < kPieces; ++u)
        if (dst[u] >= 0) out[dst[u]] = v[u];
}

}  // namespace

hipError_t launch_gather(const void* table, int64_t table_rows, int64_t row_bytes,
                         int64_t pair_stride, int P, const int32_t* idx, const int32_t* len,
                         int cap, void* out, hipStream_t st)
{
    const int64_t ppr = row_bytes / 16;
    const int64_t per_wg = 256 * kPieces;
    dim3 grid((unsigned)((cap * ppr + per_wg - 1) / per_wg), (unsigned)P);
    gather_kernel<<<grid, 256, 0, st>>>((const uint4*)table, table_rows, pair_stride, ppr, idx, len,
                                        cap, (uint4*)out);
    return hipGetLastError();
}

}  // namespace fathom

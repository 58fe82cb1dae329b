// Read-bandwidth probe: streams a buffer once (16 B per lane per load) and
// folds it into one word per workgroup, so that the memory system -- HBM, or
// the host link when the buffer is mapped pinned host memory -- is measured
// with the same kind of wide, coalesced loads the scan issues.
#include "common.h"

namespace fathom {
namespace {

__global__ __launch_bounds__(256) void read_probe_kernel(const uint4* __restrict__ src, size_t n16,
                                                         uint32_t* __restrict__ sink)
{
    uint32_t acc = 0;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
        const uint4 v = src[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    acc = (uint32_t)wave_sum_i32((int)acc);
    if (lane_id() == 0) atomicXor(&sink[blockIdx.x & 1023], acc);
}

}  // namespace

hipError_t launch_read_probe(const void* src, size_t bytes, uint32_t* sink, hipStream_t st)
{
    const size_t n16 = bytes / 16;
    read_probe_kernel<<<dim3(2048), 256, 0, st>>>((const uint4*)src, n16, sink);
    return hipGetLastError();
}

}  // namespace fathom

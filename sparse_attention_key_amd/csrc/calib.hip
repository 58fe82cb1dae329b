// Calibration statistics on the device, from the keys of a prefill
// (yeyulingfeng.com write-up of Fathom: the water-filling weights are the
// calibration variances of the stored coordinates; the rotated storage uses
// the eigenbasis of the calibration key covariance, ordered by decreasing
// variance; the calibration-domain passage notes that statistics from the
// session's own prefill keys -- one covariance per KV head -- cost under a
// millisecond at 100k tokens).
//
// Covariance: centred population covariance in float64, in two passes (mean,
// then centred products) over chunks of kChunk tokens; every chunk writes its
// partial sums and a reduction adds them in chunk order, so the result is
// deterministic.  Basis: cyclic Jacobi, one workgroup per pair, in LDS.
#include "common.h"

namespace fathom {
namespace {

constexpr int kChunk = 2048;  // tokens per partial sum
constexpr int kSub = 32;      // tokens staged in LDS at a time
constexpr int kT = 8;         // covariance tile edge per thread

template <int DTYPE>
__device__ __forceinline__ double key_at(const void* keys, size_t off)
{
    if (DTYPE == 0) return (double)((const float*)keys)[off];
    return (double)__uint_as_float((uint32_t)((const uint16_t*)keys)[off] << 16);
}

// partial[p][c][d] = sum of the chunk's keys in channel d
template <int DTYPE>
__global__ __launch_bounds__(256) void mean_partial_kernel(const void* __restrict__ keys, int64_t m,
                                                           int D, int chunks,
                                                           double* __restrict__ partial)
{
    const int p = blockIdx.y, c = blockIdx.x;
    const int64_t t0 = (int64_t)c * kChunk;
    const int64_t t1 = t0 + kChunk < m ? t0 + kChunk : m;
    __shared__ double s_part[256];
    for (int d0 = 0; d0 < D; d0 += 256 / 2) {
        // two token lanes per channel: threads [0,128) and [128,256)
        const int d = d0 + (threadIdx.x & 127), half = threadIdx.x >> 7;
        double acc = 0.0;
        if (d < D)
#pragma unroll 8
            for (int64_t t = t0 + half; t < t1; t += 2) acc += key_at<DTYPE>(keys, ((size_t)p * m + t) * D + d);
        s_part[threadIdx.x] = acc;
        __syncthreads();
        if (half == 0 && d < D)
            partial[((size_t)p * chunks + c) * D + d] = s_part[threadIdx.x] + s_part[threadIdx.x + 128];
        __syncthreads();
    }
}

// mean[p][d] = (sum over chunks, in order) / m
__global__ __launch_bounds__(128) void mean_reduce_kernel(const double* __restrict__ partial, int64_t m,
                                                          int D, int chunks, double* __restrict__ mean)
{
    const int p = blockIdx.x;
    for (int d = threadIdx.x; d < D; d += blockDim.x) {
        double s = 0.0;
        for (int c = 0; c < chunks; ++c) s += partial[((size_t)p * chunks + c) * D + d];
        mean[(size_t)p * D + d] = s / (double)m;
    }
}

// partial[p][c][i][j] = sum over the chunk's tokens of (x_i - mu_i)(x_j - mu_j).
// 256 threads hold one kT x kT tile each of the (up to) 128 x 128 matrix.
template <int DTYPE>
__global__ __launch_bounds__(256) void cov_partial_kernel(const void* __restrict__ keys, int64_t m,
                                                          int D, int chunks,
                                                          const double* __restrict__ mean,
                                                          double* __restrict__ partial)
{
    __shared__ double s_x[kSub][kMaxD];
    __shared__ double s_mu[kMaxD];
    const int p = blockIdx.y, c = blockIdx.x;
    const int64_t t0 = (int64_t)c * kChunk;
    const int64_t t1 = t0 + kChunk < m ? t0 + kChunk : m;
    for (int d = threadIdx.x; d < kMaxD; d += blockDim.x) s_mu[d] = d < D ? mean[(size_t)p * D + d] : 0.0;
    const int ti = threadIdx.x / (kMaxD / kT), tj = threadIdx.x % (kMaxD / kT);
    const int i0 = ti * kT, j0 = tj * kT;
    double acc[kT][kT];
#pragma unroll
    for (int a = 0; a < kT; ++a)
#pragma unroll
        for (int b = 0; b < kT; ++b) acc[a][b] = 0.0;
    for (int64_t s0 = t0; s0 < t1; s0 += kSub) {
        __syncthreads();  // s_mu written / previous sub-chunk consumed
        for (int e = threadIdx.x; e < kSub * kMaxD; e += blockDim.x) {
            const int r = e / kMaxD, d = e - r * kMaxD;
            const int64_t t = s0 + r;
            s_x[r][d] = (t < t1 && d < D) ? key_at<DTYPE>(keys, ((size_t)p * m + t) * D + d) - s_mu[d] : 0.0;
        }
        __syncthreads();
        for (int r = 0; r < kSub; ++r) {
            double xi[kT], xj[kT];
#pragma unroll
            for (int a = 0; a < kT; ++a) {
                xi[a] = s_x[r][i0 + a];
                xj[a] = s_x[r][j0 + a];
            }
#pragma unroll
            for (int a = 0; a < kT; ++a)
#pragma unroll
                for (int b = 0; b < kT; ++b) acc[a][b] = __builtin_fma(xi[a], xj[b], acc[a][b]);
        }
    }
    double* out = partial + ((size_t)p * chunks + c) * D * D;
#pragma unroll
    for (int a = 0; a < kT; ++a)
#pragma unroll
        for (int b = 0; b < kT; ++b)
            if (i0 + a < D && j0 + b < D) out[(size_t)(i0 + a) * D + j0 + b] = acc[a][b];
}

// Variances alone (no covariance asked for): partial[p][c][d] = the sum over
// the chunk's tokens, in order, of (x_d - mu_d)^2 -- the float64 operations
// of cov_partial_kernel's diagonal in the same order, so the variances equal
// the covariance's diagonal bit for bit, at 1/D of its arithmetic.  One
// thread per channel; a wavefront reads whole token rows.
template <int DTYPE>
__global__ __launch_bounds__(kMaxD) void var_partial_kernel(const void* __restrict__ keys, int64_t m,
                                                            int D, int chunks,
                                                            const double* __restrict__ mean,
                                                            double* __restrict__ partial)
{
    const int p = blockIdx.y, c = blockIdx.x, d = threadIdx.x;
    if (d >= D) return;
    const int64_t t0 = (int64_t)c * kChunk;
    const int64_t t1 = t0 + kChunk < m ? t0 + kChunk : m;
    const double mu = mean[(size_t)p * D + d];
    double acc = 0.0;
#pragma unroll 8
    for (int64_t t = t0; t < t1; ++t) {
        const double x = key_at<DTYPE>(keys, ((size_t)p * m + t) * D + d) - mu;
        acc = __builtin_fma(x, x, acc);
    }
    partial[((size_t)p * chunks + c) * D + d] = acc;
}

// var[p][d] = float((sum over chunks, in order) / m), as cov_reduce_kernel
// forms the diagonal
__global__ __launch_bounds__(kMaxD) void var_reduce_kernel(const double* __restrict__ partial, int64_t m,
                                                           int D, int chunks, float* __restrict__ var)
{
    const int p = blockIdx.x;
    for (int d = threadIdx.x; d < D; d += blockDim.x) {
        double s = 0.0;
        for (int c = 0; c < chunks; ++c) s += partial[((size_t)p * chunks + c) * D + d];
        var[(size_t)p * D + d] = (float)(s / (double)m);
    }
}

// cov[p] = (sum over chunks, in order) / m; var[p][d] = float(cov[p][d][d])
__global__ __launch_bounds__(256) void cov_reduce_kernel(const double* __restrict__ partial, int64_t m,
                                                         int D, int chunks, double* __restrict__ cov,
                                                         float* __restrict__ var)
{
    const int p = blockIdx.y;
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= D * D) return;
    double s = 0.0;
    for (int c = 0; c < chunks; ++c) s += partial[((size_t)p * chunks + c) * D * D + e];
    const double v = s / (double)m;
    if (cov) cov[(size_t)p * D * D + e] = v;
    const int i = e / D;
    if (var && e == i * D + i) var[(size_t)p * D + i] = (float)v;
}

// ------------------------------------------------------------------ basis

// packed upper triangle of a symmetric D x D matrix (row-major, i <= j)
__device__ __forceinline__ int tri(int i, int j, int D)
{
    if (i > j) {
        const int t = i;
        i = j;
        j = t;
    }
    return i * D - (i * (i - 1)) / 2 + (j - i);
}

// Round-robin pairing of Dp (even) indices: in round r, slot k pairs
// partner(r, k) with partner(r, Dp - 1 - k); index Dp - 1 stays in place.
__device__ __forceinline__ int rr_index(int r, int k, int Dp)
{
    if (k == Dp - 1) return Dp - 1;
    return (k + r) % (Dp - 1);
}

constexpr int kJacobiSweeps = 20;
constexpr int kJacobiThreads = 1024;

__global__ __launch_bounds__(kJacobiThreads) void jacobi_kernel(const double* __restrict__ cov, int D,
                                                     float* __restrict__ U, float* __restrict__ lam)
{
    extern __shared__ double s_dyn[];
    const int Dp = (D + 1) & ~1;            // even size; a padding index has a zero row
    const int ntri = Dp * (Dp + 1) / 2;
    double* A = s_dyn;                       // packed symmetric, Dp x Dp
    float* V = (float*)(s_dyn + ntri);       // Dp x Dp, row-major: V[row][col]
    __shared__ double s_c[kMaxD / 2], s_s[kMaxD / 2];
    __shared__ int s_i[kMaxD / 2], s_j[kMaxD / 2];
    __shared__ double s_red[kJacobiThreads / kWave * 2];
    __shared__ int s_rank[kMaxD];
    const int p = blockIdx.x;
    const double* C = cov + (size_t)p * D * D;
    for (int i = threadIdx.x; i < Dp; i += blockDim.x)
        for (int j = i; j < Dp; ++j) A[tri(i, j, Dp)] = (i < D && j < D) ? C[(size_t)i * D + j] : 0.0;
    for (int e = threadIdx.x; e < Dp * Dp; e += blockDim.x) V[e] = (e / Dp == e % Dp) ? 1.0f : 0.0f;
    __syncthreads();
    const int half = Dp / 2;
    for (int sweep = 0; sweep < kJacobiSweeps; ++sweep) {
        // stop once the off-diagonal mass is negligible against the diagonal
        double off = 0.0, dia = 0.0;
        for (int e = threadIdx.x; e < Dp * Dp; e += blockDim.x) {
            const int i = e / Dp, j = e % Dp;
            const double v = A[tri(i, j, Dp)];
            if (i < j) off += v * v;
            else if (i == j) dia += v * v;
        }
        for (int o = 32; o > 0; o >>= 1) {
            off += __shfl_xor(off, o, kWave);
            dia += __shfl_xor(dia, o, kWave);
        }
        const int wave = threadIdx.x / kWave;
        if (lane_id() == 0) {
            s_red[2 * wave] = off;
            s_red[2 * wave + 1] = dia;
        }
        __syncthreads();
        off = 0.0;
        dia = 0.0;
        for (int w = 0; w < (int)(blockDim.x / kWave); ++w) {
            off += s_red[2 * w];
            dia += s_red[2 * w + 1];
        }
        __syncthreads();
        if (!(off > 1e-24 * dia)) break;  // relative off-diagonal norm below 1e-12
        for (int r = 0; r < Dp - 1; ++r) {
            // rotations of this round: one per disjoint pair (i, j), from the
            // pair's 2 x 2 diagonal block (Rutishauser's formulas)
            for (int k = threadIdx.x; k < half; k += blockDim.x) {
                int i = rr_index(r, k, Dp), j = rr_index(r, Dp - 1 - k, Dp);
                if (i > j) {
                    const int t = i;
                    i = j;
                    j = t;
                }
                const double aij = A[tri(i, j, Dp)];
                double c = 1.0, s = 0.0;
                if (aij != 0.0) {
                    const double theta = (A[tri(j, j, Dp)] - A[tri(i, i, Dp)]) / (2.0 * aij);
                    const double t = (theta >= 0.0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(theta * theta + 1.0));
                    c = 1.0 / sqrt(t * t + 1.0);
                    s = t * c;
                }
                s_c[k] = c;
                s_s[k] = s;
                s_i[k] = i;
                s_j[k] = j;
            }
            __syncthreads();
            // A <- J^T A J: every 2 x 2 block (pair x, pair y), x <= y, on its
            // own.  The half*(half+1)/2 blocks are enumerated by folding row
            // r of the triangle (half - r blocks) with row half-1-r (r + 1
            // blocks) into one row of half + 1 (half is even when D > 2).
            const int wrow = half + 1;
            const int nblk = (half / 2) * wrow + (half & 1) * ((half + 1) / 2);
            for (int b = threadIdx.x; b < nblk; b += blockDim.x) {
                int x, y;
                const int r = b / wrow, c = b - r * wrow;
                if (r < half / 2) {
                    if (c < half - r) {
                        x = r;
                        y = r + c;
                    } else {
                        x = half - 1 - r;
                        y = x + (c - (half - r));
                    }
                } else {  // odd half: the middle row alone
                    x = half / 2;
                    y = x + c;
                }
                const int xi = s_i[x], xj = s_j[x], yi = s_i[y], yj = s_j[y];
                const double cx = s_c[x], sx = s_s[x], cy = s_c[y], sy = s_s[y];
                if (x == y) {
                    const double aii = A[tri(xi, xi, Dp)], ajj = A[tri(xj, xj, Dp)], aij = A[tri(xi, xj, Dp)];
                    A[tri(xi, xi, Dp)] = cx * cx * aii - 2.0 * sx * cx * aij + sx * sx * ajj;
                    A[tri(xj, xj, Dp)] = sx * sx * aii + 2.0 * sx * cx * aij + cx * cx * ajj;
                    A[tri(xi, xj, Dp)] = 0.0;
                } else {
                    const double a11 = A[tri(xi, yi, Dp)], a12 = A[tri(xi, yj, Dp)];
                    const double a21 = A[tri(xj, yi, Dp)], a22 = A[tri(xj, yj, Dp)];
                    // rows: [xi; xj] <- [c -s; s c] [xi; xj]
                    const double b11 = cx * a11 - sx * a21, b12 = cx * a12 - sx * a22;
                    const double b21 = sx * a11 + cx * a21, b22 = sx * a12 + cx * a22;
                    // columns: [yi yj] <- [yi yj] [c s; -s c]
                    A[tri(xi, yi, Dp)] = cy * b11 - sy * b12;
                    A[tri(xi, yj, Dp)] = sy * b11 + cy * b12;
                    A[tri(xj, yi, Dp)] = cy * b21 - sy * b22;
                    A[tri(xj, yj, Dp)] = sy * b21 + cy * b22;
                }
            }
            // V <- V J
            for (int e = threadIdx.x; e < Dp * half; e += blockDim.x) {
                const int row = e / half, k = e - row * half;
                const int i = s_i[k], j = s_j[k];
                const float c = (float)s_c[k], s = (float)s_s[k];
                const float vi = V[row * Dp + i], vj = V[row * Dp + j];
                V[row * Dp + i] = c * vi - s * vj;
                V[row * Dp + j] = s * vi + c * vj;
            }
            __syncthreads();
        }
    }
    // eigenvalues by descending value (ties by index); each eigenvector's
    // largest-magnitude component (first such) made positive
    for (int i = threadIdx.x; i < D; i += blockDim.x) {
        const double li = A[tri(i, i, Dp)];
        int rank = 0;
        for (int j = 0; j < D; ++j) {
            const double lj = A[tri(j, j, Dp)];
            rank += (lj > li || (lj == li && j < i)) ? 1 : 0;
        }
        s_rank[i] = rank;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < D; i += blockDim.x) {
        const int col = s_rank[i];
        float best = 0.0f;
        for (int row = 0; row < D; ++row) {
            const float v = V[row * Dp + i];
            if (fabsf(v) > fabsf(best)) best = v;
        }
        const float sg = best < 0.0f ? -1.0f : 1.0f;
        for (int row = 0; row < D; ++row) U[((size_t)p * D + row) * D + col] = sg * V[row * Dp + i];
        const double l = A[tri(i, i, Dp)];
        lam[(size_t)p * D + col] = l > 0.0 ? (float)l : 0.0f;
    }
}

}  // namespace

size_t calib_workspace_bytes(int P, int64_t m, int D)
{
    const int64_t chunks = (m + kChunk - 1) / kChunk;
    return (size_t)P * chunks * D * sizeof(double) * (1 + (size_t)D) + (size_t)P * D * sizeof(double);
}

hipError_t launch_calib_covariance(const void* keys, int dtype, int P, int64_t m, int D, double* cov,
                                   float* var, void* ws, hipStream_t st)
{
    const int chunks = (int)((m + kChunk - 1) / kChunk);
    double* mean = (double*)ws;
    double* mpart = mean + (size_t)P * D;
    double* cpart = mpart + (size_t)P * chunks * D;
    const dim3 grid((unsigned)chunks, (unsigned)P);
    if (!cov) {
        // variances only: the mean, then the centred squares per channel
        // (their partial sums reuse the mean's partial area)
        if (dtype == 0) {
            mean_partial_kernel<0><<<grid, 256, 0, st>>>(keys, m, D, chunks, mpart);
            mean_reduce_kernel<<<dim3((unsigned)P), 128, 0, st>>>(mpart, m, D, chunks, mean);
            var_partial_kernel<0><<<grid, kMaxD, 0, st>>>(keys, m, D, chunks, mean, mpart);
        } else {
            mean_partial_kernel<1><<<grid, 256, 0, st>>>(keys, m, D, chunks, mpart);
            mean_reduce_kernel<<<dim3((unsigned)P), 128, 0, st>>>(mpart, m, D, chunks, mean);
            var_partial_kernel<1><<<grid, kMaxD, 0, st>>>(keys, m, D, chunks, mean, mpart);
        }
        var_reduce_kernel<<<dim3((unsigned)P), kMaxD, 0, st>>>(mpart, m, D, chunks, var);
        return hipGetLastError();
    }
    if (dtype == 0) {
        mean_partial_kernel<0><<<grid, 256, 0, st>>>(keys, m, D, chunks, mpart);
        mean_reduce_kernel<<<dim3((unsigned)P), 128, 0, st>>>(mpart, m, D, chunks, mean);
        cov_partial_kernel<0><<<grid, 256, 0, st>>>(keys, m, D, chunks, mean, cpart);
    } else {
        mean_partial_kernel<1><<<grid, 256, 0, st>>>(keys, m, D, chunks, mpart);
        mean_reduce_kernel<<<dim3((unsigned)P), 128, 0, st>>>(mpart, m, D, chunks, mean);
        cov_partial_kernel<1><<<grid, 256, 0, st>>>(keys, m, D, chunks, mean, cpart);
    }
    cov_reduce_kernel<<<dim3((unsigned)((D * D + 255) / 256), (unsigned)P), 256, 0, st>>>(cpart, m, D, chunks,
                                                                                         cov, var);
    return hipGetLastError();
}

hipError_t launch_calib_basis(const double* cov, int P, int D, float* U, float* lam, hipStream_t st)
{
    const int Dp = (D + 1) & ~1;
    const size_t dyn = (size_t)Dp * (Dp + 1) / 2 * sizeof(double) + (size_t)Dp * Dp * sizeof(float);
    // set on every call (cheap next to the solve): the setting is per device
    const hipError_t e = hipFuncSetAttribute((const void*)jacobi_kernel,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
    if (e != hipSuccess) return e;
    jacobi_kernel<<<dim3((unsigned)P), kJacobiThreads, dyn, st>>>(cov, D, U, lam);
    return hipGetLastError();
}

}  // namespace fathom

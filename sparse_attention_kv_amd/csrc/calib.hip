// Reconstruction-error reduction for retention calibration (FlashLoop paper,
// App. E "Quantization Setting": the retention ratio of each loop is the
// smallest one whose hidden states stay within a relative reconstruction
// error of the reference run).
//
//  k_sq_err_part   each workgroup accumulates sum (x - ref)^2 and sum ref^2
//                  over a grid-strided slice in fp64 and writes one pair of
//                  partial sums (HBM-streaming: 8 bytes in per element).
//  k_sq_err_final  one workgroup adds the partial pairs in a fixed order.
// The grid size depends only on n, so results are deterministic.
#include "fl_device.h"
#include "fl_kernels.h"

namespace fl {

constexpr int kErrThreads = 256;

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// block-wide sum of (a, b) over 256 threads; result valid in thread 0
__device__ __forceinline__ void block_sum2(double& a, double& b) {
    __shared__ double sa[kErrThreads / 64], sb[kErrThreads / 64];
    a = wave_sum_f64(a);
    b = wave_sum_f64(b);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) { sa[w] = a; sb[w] = b; }
    __syncthreads();
    if (threadIdx.x == 0) {
        a = 0.0; b = 0.0;
        for (int i = 0; i < kErrThreads / 64; ++i) { a += sa[i]; b += sb[i]; }
    }
}

__global__ __launch_bounds__(kErrThreads) void k_sq_err_part(const float* __restrict__ x,
                                                             const float* __restrict__ ref, long n,
                                                             double* __restrict__ part) {
    double e2 = 0.0, r2 = 0.0;
    const long n4 = n / 4;
    const long stride = (long)gridDim.x * kErrThreads;
    const float4* x4 = reinterpret_cast<const float4*>(x);
    const float4* r4 = reinterpret_cast<const float4*>(ref);
    for (long i = (long)blockIdx.x * kErrThreads + threadIdx.x; i < n4; i += stride) {
        const float4 a = x4[i], b = r4[i];
        const double d0 = (double)a.x - b.x, d1 = (double)a.y - b.y;
        const double d2 = (double)a.z - b.z, d3 = (double)a.w - b.w;
        e2 += d0 * d0 + d1 * d1 + d2 * d2 + d3 * d3;
        r2 += (double)b.x * b.x + (double)b.y * b.y + (double)b.z * b.z + (double)b.w * b.w;
    }
    if (blockIdx.x == 0)
        for (long i = n4 * 4 + threadIdx.x; i < n; i += kErrThreads) {
            const double d = (double)x[i] - ref[i];
            e2 += d * d;
            r2 += (double)ref[i] * ref[i];
        }
    block_sum2(e2, r2);
    if (threadIdx.x == 0) {
        part[2 * blockIdx.x] = e2;
        part[2 * blockIdx.x + 1] = r2;
    }
}

__global__ __launch_bounds__(kErrThreads) void k_sq_err_final(const double* __restrict__ part,
                                                              int nb, double* __restrict__ out) {
    double e2 = 0.0, r2 = 0.0;
    for (int i = threadIdx.x; i < nb; i += kErrThreads) {
        e2 += part[2 * i];
        r2 += part[2 * i + 1];
    }
    block_sum2(e2, r2);
    if (threadIdx.x == 0) { out[0] = e2; out[1] = r2; }
}

int sq_err_blocks(long n) {
    const long per = (long)kErrThreads * 4 * 16; // >= 16 float4 per thread before growing
    long b = (n + per - 1) / per;
    if (b < 1) b = 1;
    if (b > 2048) b = 2048;
    return (int)b;
}

hipError_t launch_sq_err(const float* x, const float* ref, long n, double* part, double* out,
                         hipStream_t st) {
    const int nb = sq_err_blocks(n);
    hipLaunchKernelGGL(k_sq_err_part, dim3(nb), dim3(kErrThreads), 0, st, x, ref, n, part);
    hipLaunchKernelGGL(k_sq_err_final, dim3(1), dim3(kErrThreads), 0, st, part, nb, out);
    return hipGetLastError();
}

} // namespace fl

// The balance statistics as a kernel of their own (balance_stats.h) for moe_balance_stats (the
// layer forward computes them in an extra block of its combine launch), and a plain fp32 copy.
#include "balance_stats.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void stats_kernel(
    int64_t T, int E, double fden, const int32_t* __restrict__ n, const double* __restrict__ gsum,
    const double* __restrict__ lse2sum, const double* __restrict__ hsum, float lambda,
    float* __restrict__ f, float* __restrict__ P, float* __restrict__ aux, float* __restrict__ z,
    float* __restrict__ diag, const float* __restrict__ b, float* __restrict__ b_new,
    float gamma) {
  balance_stats<256>(T, E, fden, n, gsum, lse2sum, hsum, lambda, f, P, aux, z, diag, b, b_new,
                     gamma);
}

__global__ __launch_bounds__(256) void copy_f32_kernel(const float* __restrict__ src,
                                                        float* __restrict__ dst, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src != nullptr ? src[i] : 0.f;
}

}  // namespace

hipError_t launch_copy_f32(const float* src, float* dst, int n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(copy_f32_kernel, dim3((n + 255) / 256), dim3(256), 0, st, src, dst, n);
  return hipGetLastError();
}

hipError_t launch_stats(int64_t T, int E, double fden, const int32_t* n, const double* gsum,
                        const double* lse2sum, const double* hsum, float lambda, float* f,
                        float* P, float* aux, float* z, float* diag, const float* b, float* b_new,
                        float gamma, hipStream_t st) {
  hipLaunchKernelGGL(stats_kernel, dim3(1), dim3(256), 0, st, T, E, fden, n, gsum, lse2sum, hsum,
                     lambda, f, P, aux, z, diag, b, b_new, gamma);
  return hipGetLastError();
}

}  // namespace moe

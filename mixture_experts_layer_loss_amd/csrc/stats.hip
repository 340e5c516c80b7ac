// Balance statistics and the loss-free-balancing bias step, from the reduced route statistics:
//   f_e = n_e / (k T), P_e = gsum_e / T, aux = lambda E sum_e f_e P_e
//   ("MoE：条件计算与路由" §原理与演进; "深入理解 MoE (混合专家模型)：稀疏激活与高效扩展" §4.2.1;
//   "MOE大模型对比篇" §2.1), z = lse2sum / T ("MOE大模型对比篇" §2.2), and
//   b_e <- b_e + gamma * sign(k T / E - n_e) ("MoE：条件计算与路由" §无辅助损失负载均衡（ALF-LB）).
// One block; fp64 inside, the sum over experts is a fixed-order tree, outputs are fp32. The sign
// compares the integers k T and n_e E, so it is exact; the bias step is a single fp32 addition of
// +-gamma or 0.
#include "moe_internal.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void stats_kernel(int64_t T, int E, int k,
                                                     const int32_t* __restrict__ n,
                                                     const double* __restrict__ gsum,
                                                     const double* __restrict__ lse2sum,
                                                     float lambda, float* __restrict__ f,
                                                     float* __restrict__ P, float* __restrict__ aux,
                                                     float* __restrict__ z,
                                                     const float* __restrict__ b,
                                                     float* __restrict__ b_new, float gamma) {
  __shared__ double red[256];
  const int e = threadIdx.x;
  double prod = 0.0;
  float bnew = 0.f;
  if (e < E) {
    const double fe = static_cast<double>(n[e]) / (static_cast<double>(k) * static_cast<double>(T));
    const double pe = gsum[e] / static_cast<double>(T);
    prod = fe * pe;
    if (f != nullptr) f[e] = static_cast<float>(fe);
    if (P != nullptr) P[e] = static_cast<float>(pe);
    if (b != nullptr) {
      const int64_t kt = static_cast<int64_t>(k) * T, ne = static_cast<int64_t>(n[e]) * E;
      const float sgn = kt > ne ? 1.f : (kt < ne ? -1.f : 0.f);
      bnew = b[e] + gamma * sgn;
    }
  }
  red[e] = prod;
  __syncthreads();  // every read of b is done before any write of b_new (they may alias)
  if (e < E && b_new != nullptr) b_new[e] = bnew;
  for (int off = 128; off >= 1; off >>= 1) {
    if (e < off) red[e] += red[e + off];
    __syncthreads();
  }
  if (e == 0) {
    if (aux != nullptr) *aux = static_cast<float>(static_cast<double>(lambda) * E * red[0]);
    if (z != nullptr) *z = static_cast<float>(*lse2sum / static_cast<double>(T));
  }
}

}  // namespace

hipError_t launch_stats(int64_t T, int E, int k, const int32_t* n, const double* gsum,
                        const double* lse2sum, float lambda, float* f, float* P, float* aux,
                        float* z, const float* b, float* b_new, float gamma, hipStream_t st) {
  hipLaunchKernelGGL(stats_kernel, dim3(1), dim3(256), 0, st, T, E, k, n, gsum, lse2sum, lambda, f,
                     P, aux, z, b, b_new, gamma);
  return hipGetLastError();
}

}  // namespace moe

// Balance statistics and the loss-free-balancing bias step, from the reduced route statistics:
//   f_e = n_e / (k T) (token choice; expert choice: n_e / (E r)), P_e = gsum_e / T,
//   aux = lambda E sum_e f_e P_e
//   ("MoE：条件计算与路由" §原理与演进; "深入理解 MoE (混合专家模型)：稀疏激活与高效扩展" §4.2.1;
//   "MOE大模型对比篇" §2.1), z = lse2sum / T ("MOE大模型对比篇" §2.2), and
//   b_e <- b_e + gamma * sign(k T / E - n_e) ("MoE：条件计算与路由" §无辅助损失负载均衡（ALF-LB）).
// Routing diagnostics ("MoE：条件计算与路由" §9 routing entropy, §10 load Gini coefficient and
// max/mean load; the adg.csdn.net notes page, importance CV^2 of Importance_e = gsum_e):
//   entropy = hsum / T, Gini = sum_ij |n_i - n_j| / (2 E sum_e n_e) (integer sums, exact),
//   max/mean = max_e n_e E / sum_e n_e, CV^2 = Var_e(gsum) / Mean_e(gsum)^2 (population variance).
// Computed by NTH threads of one block (E <= NTH <= 1024, a multiple of 64), every one of which must
// call it (it has barriers); fp64 inside, sums over experts are fixed-order trees, outputs are fp32. The sign
// compares the integers k T and n_e E, so it is exact; the bias step is a single fp32 addition of
// +-gamma or 0.
#pragma once
#include "moe_internal.h"

namespace moe {

template <int NTH>
__device__ __forceinline__ void balance_stats(
    int64_t T, int E, double fden, const int32_t* __restrict__ n, const double* __restrict__ gsum,
    const double* __restrict__ lse2sum, const double* __restrict__ hsum, float lambda,
    float* __restrict__ f, float* __restrict__ P, float* __restrict__ aux, float* __restrict__ z,
    float* __restrict__ diag, const float* __restrict__ b, float* __restrict__ b_new,
    float gamma) {
  __shared__ double wsum[NTH / 64];
  __shared__ long long wisum[NTH / 64];
  const int e = threadIdx.x, lane = e & 63, wave = e >> 6;
  // fixed-order sums over the threads (every thread returns the total): a butterfly inside each
  // wave, then the wave sums in wave order (threads past E add zeros, so the sums do not depend
  // on NTH)
  auto tree = [&](double v) -> double {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    if (lane == 0) wsum[wave] = v;
    __syncthreads();
    double r = wsum[0];
    for (int w = 1; w < NTH / 64; ++w) r += wsum[w];
    __syncthreads();
    return r;
  };
  auto itree = [&](long long v, bool take_max) -> long long {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const long long o = __shfl_xor(v, off, 64);
      v = take_max ? max(v, o) : v + o;
    }
    if (lane == 0) wisum[wave] = v;
    __syncthreads();
    long long r = wisum[0];
    for (int w = 1; w < NTH / 64; ++w) r = take_max ? max(r, wisum[w]) : r + wisum[w];
    __syncthreads();
    return r;
  };
  __shared__ int nl[NTH];  // the loads, for the pairwise Gini sum
  const long long ne = e < E ? n[e] : 0;
  nl[e] = static_cast<int>(ne);
  double prod = 0.0;
  float bnew = 0.f;
  if (e < E) {
    const double fe = static_cast<double>(n[e]) / fden;
    const double pe = gsum[e] / static_cast<double>(T);
    prod = fe * pe;
    if (f != nullptr) f[e] = static_cast<float>(fe);
    if (P != nullptr) P[e] = static_cast<float>(pe);
    if (b != nullptr) {
      // sign(k T / E - n_e) as an integer comparison of k T and n_e E (fden = k T here)
      const int64_t kt = static_cast<int64_t>(fden), nE = static_cast<int64_t>(n[e]) * E;
      const float sgn = kt > nE ? 1.f : (kt < nE ? -1.f : 0.f);
      bnew = b[e] + gamma * sgn;
    }
  }
  __syncthreads();  // every read of b is done before any write of b_new (they may alias)
  if (e < E && b_new != nullptr) b_new[e] = bnew;
  const double fp = tree(prod);
  if (e == 0) {
    if (aux != nullptr) *aux = static_cast<float>(static_cast<double>(lambda) * E * fp);
    if (z != nullptr) *z = static_cast<float>(*lse2sum / static_cast<double>(T));
  }
  if (diag == nullptr) return;
  // Gini: sum over pairs of |n_i - n_j| (integers), over 2 E sum_e n_e
  long long pairs = 0;
  if (e < E)
#pragma unroll 8
    for (int j = 0; j < E; ++j) {
      const long long d = ne - static_cast<long long>(nl[j]);
      pairs += d < 0 ? -d : d;
    }
  const long long psum = itree(pairs, false);
  const long long ntot = itree(ne, false);
  const long long nmax = itree(ne, true);
  // importance CV^2: population variance over experts of gsum, over the squared mean
  const double imp = e < E ? gsum[e] : 0.0;
  const double mean = tree(imp) / E;
  const double dv = e < E ? imp - mean : 0.0;
  const double var = tree(dv * dv) / E;
  if (e == 0) {
    diag[0] = static_cast<float>(*hsum / static_cast<double>(T));
    diag[1] = ntot > 0 ? static_cast<float>(static_cast<double>(psum) / (2.0 * E * ntot)) : 0.f;
    diag[2] = ntot > 0 ? static_cast<float>(static_cast<double>(nmax) * E / ntot) : 0.f;
    diag[3] = mean != 0.0 ? static_cast<float>(var / (mean * mean)) : 0.f;
  }
}

}  // namespace moe

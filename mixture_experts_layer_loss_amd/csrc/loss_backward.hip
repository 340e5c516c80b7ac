// Backward of the layer's balance losses through the router: L = aux + z_coef z with
// aux = lambda E sum_e f_e P_e and z = mean_t lse_t^2 ("MoE：条件计算与路由" §原理与演进: f_e counts
// discrete choices, so the gradient reaches the router through P_e; "MOE大模型对比篇" §2.2 z-loss).
// With a_e = lambda E f_e / T, f held fixed:
//   softmax scores (p = g):   dL/dl_te = g_te (a_e - sum_e' g_te' a_e') + z_coef (2/T) lse_t g_te
//   sigmoid scores (p = s/S): dL/dl_te = s_te (1 - s_te) (a_e - sum_e' p_te' a_e') / S_t
//                                        + z_coef (2/T) lse_t softmax(l_t)_e
// then dW_r = dl^T x and dx = dl W_r.
//   loss_grad_kernel: one wave per token over the expert-major logit/score columns the router
//   writes in its column mode; fixed butterfly reductions (reproducible); dl leaves in both
//   [T][E] and [E][T] layouts, so that both products below read K-major operands.
//   kmajor_gemm_kernel: C[M][N] = sum_k A[k][m] B[k][n] with fp32 A and bf16/fp32 B, both stored
//   K-major; 64 x 64 tiles, 256 threads with 4 x 4 outputs each, K staged 16 at a time in LDS,
//   fp32 accumulation in k order. A long K (dW_r sums over all T tokens) is split into KS ranges
//   whose partial tiles are summed afterwards in range order (reproducible). (These products
//   are ~1% of the forward's flops.)
#include "moe_internal.h"

#include <math.h>

namespace moe {
namespace {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

constexpr int kEPL = MOE_E_MAX / 64;  // experts per lane

__global__ __launch_bounds__(256) void loss_grad_kernel(int64_t T, int E, int sigmoid,
                                                         const float* __restrict__ lcol,
                                                         const float* __restrict__ scol,
                                                         const int32_t* __restrict__ n,
                                                         double fden, float lambda, float z_coef,
                                                         float* __restrict__ dl,
                                                         float* __restrict__ dlT) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float l[kEPL], s[kEPL], a[kEPL];
  float m = -INFINITY;
#pragma unroll
  for (int q = 0; q < kEPL; ++q) {
    const int e = lane + 64 * q;
    const bool in = e < E;
    l[q] = in ? lcol[static_cast<int64_t>(e) * T + t] : -INFINITY;
    s[q] = in ? scol[static_cast<int64_t>(e) * T + t] : 0.f;
    a[q] = in ? static_cast<float>(static_cast<double>(lambda) * E *
                                   (static_cast<double>(n[e]) / fden) / static_cast<double>(T))
              : 0.f;
    m = fmaxf(m, l[q]);
  }
  m = wave_max(m);
  float se = 0.f;
#pragma unroll
  for (int q = 0; q < kEPL; ++q) se += expf(l[q] - m);  // the pad adds exp(-inf) = 0
  const float lse = m + logf(wave_sum(se));
  const float zc = z_coef * 2.f * lse / static_cast<float>(T);
  float S = 1.f, c = 0.f;
  if (sigmoid) {
    float ss = 0.f;
#pragma unroll
    for (int q = 0; q < kEPL; ++q) ss += s[q];
    S = wave_sum(ss);
  }
  float ca = 0.f;
#pragma unroll
  for (int q = 0; q < kEPL; ++q) ca += s[q] * a[q];
  c = wave_sum(ca) / S;  // sum_e p_e a_e (softmax: S = 1)
#pragma unroll
  for (int q = 0; q < kEPL; ++q) {
    const int e = lane + 64 * q;
    if (e < E) {
      const float soft = expf(l[q] - lse);
      const float g = sigmoid ? s[q] * (1.f - s[q]) * (a[q] - c) / S : s[q] * (a[q] - c);
      const float v = g + zc * soft;
      dl[t * E + e] = v;
      dlT[static_cast<int64_t>(e) * T + t] = v;
    }
  }
}

template <typename TB>
__device__ __forceinline__ float to_f32(TB v);
template <>
__device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v); }

constexpr int GM = 64, GN = 64, GK = 16;

// blockIdx.y = K range ks of KS (each kc long, a multiple of GK); its partial tile goes to
// C + ks M N (KS = 1: the result itself)
template <typename TB>
__global__ __launch_bounds__(256) void kmajor_gemm_kernel(int64_t M, int64_t N, int64_t K,
                                                           int64_t kc,
                                                           const float* __restrict__ A,
                                                           const TB* __restrict__ B,
                                                           float* __restrict__ C) {
  __shared__ float As[GK][GM + 4];
  __shared__ float Bs[GK][GN + 4];
  const int64_t nb = (N + GN - 1) / GN;
  const int64_t m0 = static_cast<int64_t>(blockIdx.x / nb) * GM;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x % nb) * GN;
  const int64_t kbeg = static_cast<int64_t>(blockIdx.y) * kc;
  const int64_t kend = min(K, kbeg + kc);
  C += static_cast<int64_t>(blockIdx.y) * M * N;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {};
  for (int64_t k0 = kbeg; k0 < kend; k0 += GK) {
    for (int c = tid; c < GK * GM; c += 256) {
      const int kk = c / GM, mm = c % GM;
      const int64_t k = k0 + kk, m = m0 + mm;
      As[kk][mm] = (k < kend && m < M) ? A[k * M + m] : 0.f;
    }
    for (int c = tid; c < GK * GN; c += 256) {
      const int kk = c / GN, nn = c % GN;
      const int64_t k = k0 + kk, n = n0 + nn;
      Bs[kk][nn] = (k < kend && n < N) ? to_f32<TB>(B[k * N + n]) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < GK; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + ty * 4 + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + tx * 4 + j;
      if (n < N) C[m * N + n] = acc[i][j];
    }
  }
}

// C[i] = sum_s P[s][i] in s order
__global__ __launch_bounds__(256) void sum_ranges_kernel(int64_t count, int KS,
                                                          const float* __restrict__ P,
                                                          float* __restrict__ C) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= count) return;
  float v = 0.f;
  for (int s = 0; s < KS; ++s) v += P[s * count + i];
  C[i] = v;
}

template <typename TB>
hipError_t launch_kmajor(int64_t M, int64_t N, int64_t K, int KS, const float* A, const void* B,
                         float* C, float* partial, hipStream_t st) {
  const int64_t tiles = ((M + GM - 1) / GM) * ((N + GN - 1) / GN);
  if (tiles == 0) return hipSuccess;
  if (tiles > 0x7fffffff) return hipErrorInvalidValue;
  const int64_t kc = ((cdiv(K, KS) + GK - 1) / GK) * GK;
  hipLaunchKernelGGL(kmajor_gemm_kernel<TB>, dim3(static_cast<unsigned>(tiles), KS), dim3(256), 0,
                     st, M, N, K, kc, A, static_cast<const TB*>(B), KS > 1 ? partial : C);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || KS == 1) return e;
  hipLaunchKernelGGL(sum_ranges_kernel, dim3(static_cast<unsigned>(cdiv(M * N, 256))), dim3(256),
                     0, st, M * N, KS, partial, C);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sum_ranges(int64_t count, int KS, const float* P, float* C, hipStream_t st) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(sum_ranges_kernel, dim3(static_cast<unsigned>(cdiv(count, 256))), dim3(256),
                     0, st, count, KS, P, C);
  return hipGetLastError();
}

hipError_t launch_loss_grad(int64_t T, int E, int sigmoid, const float* lcol, const float* scol,
                            const int32_t* n, double fden, float lambda, float z_coef, float* dl,
                            float* dlT, hipStream_t st) {
  hipLaunchKernelGGL(loss_grad_kernel, dim3(static_cast<unsigned>(cdiv(T, 4))), dim3(256), 0, st,
                     T, E, sigmoid, lcol, scol, n, fden, lambda, z_coef, dl, dlT);
  return hipGetLastError();
}

int kmajor_splits(int64_t M, int64_t N, int64_t K) {
  // enough K ranges for ~1024 blocks, each range at least 256 long
  const int64_t tiles = ((M + GM - 1) / GM) * ((N + GN - 1) / GN);
  int64_t ks = cdiv(1024, tiles);
  const int64_t by_len = K / 256 > 1 ? K / 256 : 1;
  if (ks > by_len) ks = by_len;
  if (ks > 64) ks = 64;
  return static_cast<int>(ks < 1 ? 1 : ks);
}

hipError_t launch_kmajor_gemm(int dtype_b, int64_t M, int64_t N, int64_t K, int KS, const float* A,
                              const void* B, float* C, float* partial, hipStream_t st) {
  return dtype_b == MOE_F32 ? launch_kmajor<float>(M, N, K, KS, A, B, C, partial, st)
                            : launch_kmajor<bf16_t>(M, N, K, KS, A, B, C, partial, st);
}

}  // namespace moe

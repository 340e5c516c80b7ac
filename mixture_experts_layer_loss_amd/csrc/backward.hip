// Backward of the layer: gradients of <dy, y> + aux + z_coef z with respect to x, W_r and every
// expert weight, with the selection, the capacity cut and f held fixed (they are discrete). The
// chain ("MoE：条件计算与路由" §7 eqs. (1)-(3) for y and the gates; "深入理解 MoE
// (混合专家模型)：稀疏激活与高效扩展" §10.2 for SwiGLU; the balance-loss part as in
// loss_backward.hip):
//   combine:  d out[row(t,j)] = w_tj dy_t,  d w_tj = <dy_t, out[row(t,j)]> = <dy_t W_down[e], h>
//             (kept slots; P_row = dy_t W_down[e] is formed once and gives both d w and dh)
//   gates:    renorm: dg_e = (dw_e - sum_j w_j dw_j) / sum_S g;  else dg_e = dw_e   (e in S_t)
//   scores:   softmax dl = g (dg - sum_e g dg);  sigmoid dl = s (1 - s) dg;  + balance-loss term
//   down:     dh = w_tj P_row,  dW_down[e] = sum_rows d out^T h
//   SwiGLU:   dG = dh U SiLU'(G),  dU = dh SiLU(G),  SiLU'(z) = sigma(z) (1 + z (1 - sigma(z)))
//   up:       dx_row = dG W_gate[e] + dU W_up[e],  dW_gate[e] = sum_rows dG^T x,  dW_up likewise
//   tokens:   dx_t = (dl W_r)_t + sum_j dx_row(t,j) (slot order) + shared experts' dx_t
// Under expert choice the slots of token t are the experts that took it (ascending), read from the
// row map. The pre-activations G, U are recomputed in fp32 and h = SiLU(G) U is formed in fp32 from
// them, so the gradients follow the real-valued chain (the forward's bf16 roundings of h and of the
// expert outputs are not differentiated).
// This file holds the per-row, per-token and elementwise kernels, and the fp32 SIMT products used
// by fp32 layers (64 x 64 outputs, 256 threads, 4 x 4 each, K staged 16 at a time in LDS,
// accumulation in k order): "NN" products read A row-major and the weight K-major (B[k][n]); weight
// gradients reduce over a group's rows with both operands K-major (rows), the x operand gathered
// through perm_token; groups never share a 64-row tile. bf16 layers run the products on the MFMA
// grouped GEMM instead (gemm_bf16.hip, operand layouts from backward_layout.hip).
#include "moe_internal.h"

#include <math.h>

namespace moe {
namespace {

template <typename T>
__device__ __forceinline__ float ld(const T* p, int64_t i);
template <>
__device__ __forceinline__ float ld<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld<bf16_t>(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i]); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Per kept row (one wave): t = perm_token[row], its slot j and gate w. From P_row = dy_t W_down[e]
// and the fp32 pre-activations G, U of the row: h = SiLU(G) U, d w_tj = <P_row, h>, dh = w P_row,
// and the SwiGLU derivative dG = dh U SiLU'(G), dU = dh SiLU(G) with SiLU'(z) = s (1 + z (1 - s)),
// s = sigma(z). CAT: one bf16 row [dG | dU] of 2M (M a multiple of 4; lanes take 4 columns at a
// time); else fp32 rows dG, dU. When not NULL: d out_row = w dy_t, wrow[row] = w.
// Expert choice (inv_perm == NULL): the row's gate is read from wrow and d w is written per row,
// dw[row].
template <typename T, bool CAT>
__global__ __launch_bounds__(256) void bw_rows_kernel(
    const int32_t* __restrict__ offsets, int E, int d, int M, int k,
    const int32_t* __restrict__ perm_token, const int32_t* __restrict__ inv_perm,
    const float* __restrict__ topk_w, const T* __restrict__ dy, const float* __restrict__ P,
    const float* __restrict__ G, const float* __restrict__ U, float* __restrict__ dw,
    float* __restrict__ dG, float* __restrict__ dU, bf16_t* __restrict__ dGU,
    bf16_t* __restrict__ wh, float* __restrict__ dout, float* __restrict__ wrow) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= offsets[E]) return;
  const int64_t t = perm_token[row];
  const bool ec = inv_perm == nullptr;
  int slot = 0;
  if (!ec)
    for (int j = 0; j < k; ++j)
      if (inv_perm[t * k + j] == row) slot = j;
  const float w = ec ? wrow[row] : topk_w[t * k + slot];
  float dot = 0.f;
  auto one = [&](float p, float z, float u, float& vg, float& vu) __attribute__((always_inline)) {
    const float sg = 1.f / (1.f + expf(-z));
    const float si = z * sg;
    dot = fmaf(p, si * u, dot);
    const float gh = w * p;
    vg = gh * u * sg * (1.f + z * (1.f - sg));
    vu = gh * si;
  };
  if constexpr (CAT) {
    for (int m = lane * 4; m < M; m += 256) {
      const int64_t i = row * M + m;
      const float4 p = *reinterpret_cast<const float4*>(P + i);
      const float4 z = *reinterpret_cast<const float4*>(G + i);
      const float4 u = *reinterpret_cast<const float4*>(U + i);
      float vg[4], vu[4];
      one(p.x, z.x, u.x, vg[0], vu[0]);
      one(p.y, z.y, u.y, vg[1], vu[1]);
      one(p.z, z.z, u.z, vg[2], vu[2]);
      one(p.w, z.w, u.w, vg[3], vu[3]);
      const uint2 og = make_uint2(
          static_cast<uint32_t>(f32_to_bf16(vg[0])) | (static_cast<uint32_t>(f32_to_bf16(vg[1])) << 16),
          static_cast<uint32_t>(f32_to_bf16(vg[2])) | (static_cast<uint32_t>(f32_to_bf16(vg[3])) << 16));
      const uint2 ou = make_uint2(
          static_cast<uint32_t>(f32_to_bf16(vu[0])) | (static_cast<uint32_t>(f32_to_bf16(vu[1])) << 16),
          static_cast<uint32_t>(f32_to_bf16(vu[2])) | (static_cast<uint32_t>(f32_to_bf16(vu[3])) << 16));
      *reinterpret_cast<uint2*>(dGU + row * 2 * M + m) = og;
      *reinterpret_cast<uint2*>(dGU + row * 2 * M + M + m) = ou;
      if (wh != nullptr) {  // w SiLU(G) U, rounded once: an operand of dW_down
        const float zz[4] = {z.x, z.y, z.z, z.w}, uu[4] = {u.x, u.y, u.z, u.w};
        float hv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          hv[q] = zz[q] / (1.f + expf(-zz[q])) * uu[q];
          hv[q] *= w;
        }
        *reinterpret_cast<uint2*>(wh + row * M + m) = make_uint2(
            static_cast<uint32_t>(f32_to_bf16(hv[0])) | (static_cast<uint32_t>(f32_to_bf16(hv[1])) << 16),
            static_cast<uint32_t>(f32_to_bf16(hv[2])) | (static_cast<uint32_t>(f32_to_bf16(hv[3])) << 16));
      }
    }
  } else {
    for (int m = lane; m < M; m += 64) {
      const int64_t i = row * M + m;
      float vg, vu;
      one(P[i], G[i], U[i], vg, vu);
      dG[i] = vg;
      dU[i] = vu;
    }
  }
  if (dout != nullptr)
    for (int i = lane; i < d; i += 64) dout[row * d + i] = w * ld<T>(dy, t * d + i);
  dot = wave_sum(dot);
  if (lane == 0) {
    if (ec) {
      dw[row] = dot;
    } else {
      dw[t * k + slot] = dot;
      if (wrow != nullptr) wrow[row] = w;
    }
  }
}

// h = SiLU(G) U in fp32
__global__ __launch_bounds__(256) void swiglu_fwd_kernel(int64_t count, const float* __restrict__ G,
                                                          const float* __restrict__ U,
                                                          float* __restrict__ h) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= count) return;
  const float z = G[i];
  h[i] = z / (1.f + expf(-z)) * U[i];
}

constexpr int kEPL = MOE_E_MAX / 64;

// Router tail shared by both routings, one wave per token t: from dg (the gradient at the chosen
// experts' gates, lane-strided like the columns), the logits and scores: dl = the softmax or sigmoid
// chain plus the balance-loss gradient, written to dl [T][E] and dlT [E][T].
__device__ __forceinline__ void router_tail(int64_t T, int E, int sigmoid, int64_t t, int lane,
                                            const float* __restrict__ lcol,
                                            const float* __restrict__ scol,
                                            const int32_t* __restrict__ n, double fden,
                                            float lambda, float z_coef, const float* dg,
                                            float* __restrict__ dl, float* __restrict__ dlT) {
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
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  float se = 0.f, S = 0.f, ca = 0.f, cg = 0.f;
#pragma unroll
  for (int q = 0; q < kEPL; ++q) {
    se += expf(l[q] - m);
    S += s[q];
    ca += s[q] * a[q];
    cg += s[q] * dg[q];
  }
  const float lse = m + logf(wave_sum(se));
  S = sigmoid ? wave_sum(S) : 1.f;
  const float c = wave_sum(ca) / S;
  cg = wave_sum(cg);
  const float zc = z_coef * 2.f * lse / static_cast<float>(T);
#pragma unroll
  for (int q = 0; q < kEPL; ++q) {
    const int e = lane + 64 * q;
    if (e < E) {
      const float soft = expf(l[q] - lse);
      float v = sigmoid ? s[q] * (1.f - s[q]) * ((a[q] - c) / S + dg[q])
                        : s[q] * ((a[q] - c) + (dg[q] - cg));
      v += zc * soft;
      dl[t * E + e] = v;
      dlT[static_cast<int64_t>(e) * T + t] = v;
    }
  }
}

// router (token choice): gates -> scores -> logits, plus the balance-loss gradient; one wave per
// token
__global__ __launch_bounds__(256) void bw_router_kernel(
    int64_t T, int E, int k, int renorm, int sigmoid, const float* __restrict__ lcol,
    const float* __restrict__ scol, const int32_t* __restrict__ topk_idx,
    const int32_t* __restrict__ inv_perm, const float* __restrict__ topk_w,
    const float* __restrict__ dw, const int32_t* __restrict__ n,
    double fden, float lambda, float z_coef, float* __restrict__ dl, float* __restrict__ dlT) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  // dg over the chosen experts (wave-uniform, slot order)
  // d w of a dropped slot is 0 (it adds nothing to y)
  float gsel = 0.f, wdw = 0.f;
  for (int j = 0; j < k; ++j) {
    const int e = topk_idx[t * k + j];
    const float dwj = inv_perm[t * k + j] >= 0 ? dw[t * k + j] : 0.f;
    gsel += scol[static_cast<int64_t>(e) * T + t];
    wdw += topk_w[t * k + j] * dwj;
  }
  float dg[kEPL];
#pragma unroll
  for (int q = 0; q < kEPL; ++q) dg[q] = 0.f;
  for (int j = 0; j < k; ++j) {
    const int e = topk_idx[t * k + j];
    const float dwj = inv_perm[t * k + j] >= 0 ? dw[t * k + j] : 0.f;
    const float v = renorm ? (dwj - wdw) / gsel : dwj;
#pragma unroll
    for (int q = 0; q < kEPL; ++q)
      if (e == lane + 64 * q) dg[q] = v;
  }
  router_tail(T, E, sigmoid, t, lane, lcol, scol, n, fden, lambda, z_coef, dg, dl, dlT);
}

// Expert choice: the experts that took token t are those with row_of[e][t] >= 0 (lane-strided);
// gates w = g / sum over them of g (renorm; the sum taken in ascending expert order, as the
// combine does) or g. GATES: write wrow[row] = w for every taken expert. Otherwise: the router
// backward from the per-row d w (dw[row]).
template <bool GATES>
__global__ __launch_bounds__(256) void ec_token_kernel(
    int64_t T, int E, int renorm, int sigmoid, const int32_t* __restrict__ row_of,
    const float* __restrict__ lcol, const float* __restrict__ scol, float* __restrict__ wrow,
    const float* __restrict__ dw, const int32_t* __restrict__ n, double fden, float lambda,
    float z_coef, float* __restrict__ dl, float* __restrict__ dlT) {
  __shared__ float lg[4][MOE_E_MAX];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  if (t >= T) return;  // whole waves only: no block barrier below
  int row[kEPL];
  float g[kEPL];
#pragma unroll
  for (int q = 0; q < kEPL; ++q) {
    const int e = lane + 64 * q;
    row[q] = e < E ? row_of[static_cast<int64_t>(e) * T + t] : -1;
    g[q] = row[q] >= 0 ? scol[static_cast<int64_t>(e) * T + t] : 0.f;
    if (e < E) lg[wave][e] = g[q];
  }
  __builtin_amdgcn_wave_barrier();
  // the gate denominator in ascending expert order (lane 0), as in the combine
  float den = 0.f;
  if (lane == 0)
    for (int e = 0; e < E; ++e) den += lg[wave][e];
  den = __shfl(den, 0, 64);
  den = renorm && den > 0.f ? den : 1.f;
  if constexpr (GATES) {
#pragma unroll
    for (int q = 0; q < kEPL; ++q)
      if (row[q] >= 0) wrow[row[q]] = g[q] / den;
    return;
  } else {
    float dwq[kEPL], wdw = 0.f;
#pragma unroll
    for (int q = 0; q < kEPL; ++q) {
      dwq[q] = row[q] >= 0 ? dw[row[q]] : 0.f;
      wdw += (g[q] / den) * dwq[q];
    }
    wdw = wave_sum(wdw);
    float dg[kEPL];
#pragma unroll
    for (int q = 0; q < kEPL; ++q)
      dg[q] = row[q] < 0 ? 0.f : (renorm ? (dwq[q] - wdw) / den : dwq[q]);
    router_tail(T, E, sigmoid, t, lane, lcol, scol, n, fden, lambda, z_coef, dg, dl, dlT);
  }
}

constexpr int BMt = 64, BNt = 64, BKt = 16;

__device__ __forceinline__ int find_group64(const int32_t* __restrict__ table, int groups,
                                            int nb, int64_t L) {
  int lo = 0, hi = groups;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (static_cast<int64_t>(table[mid]) * nb <= L) lo = mid; else hi = mid;
  }
  return lo;
}

// C[r][n] = sum_k A[r][k] B_g[k][n] (+ A2[r][k] B2_g[k][n]) for the rows r of group g
template <typename TA, typename TB, bool TWO>
__global__ __launch_bounds__(256) void nn_gemm_kernel(
    const TA* __restrict__ A, const TA* __restrict__ A2, const int32_t* __restrict__ gather_a,
    const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ tile_off, int groups, const TB* __restrict__ B,
    const TB* __restrict__ B2, int64_t gstride, int N, int K, float* __restrict__ C) {
  __shared__ float As[BKt][BMt + 4];
  __shared__ float Bs[BKt][BNt + 4];
  const int nb = (N + BNt - 1) / BNt;
  const int64_t L = blockIdx.x;
  if (L >= static_cast<int64_t>(tile_off[groups]) * nb) return;
  const int g = find_group64(tile_off, groups, nb, L);
  const int mt_g = tile_off[g + 1] - tile_off[g];
  const int64_t local = L - static_cast<int64_t>(tile_off[g]) * nb;
  const int n0 = static_cast<int>(local / mt_g) * BNt;
  const int r0 = offsets[g] + static_cast<int>(local % mt_g) * BMt;
  const int r1 = min(r0 + BMt, offsets[g + 1]);
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {};
  for (int pass = 0; pass < (TWO ? 2 : 1); ++pass) {
    const TA* Ap = pass == 0 ? A : A2;
    const TB* Bp = (pass == 0 ? B : B2) + static_cast<int64_t>(g) * gstride;
    for (int k0 = 0; k0 < K; k0 += BKt) {
      for (int c = tid; c < BKt * BMt; c += 256) {
        const int mm = c / BKt, kk = c % BKt;
        const int r = r0 + mm, kx = k0 + kk;
        float v = 0.f;
        if (r < r1 && kx < K) {
          const int64_t ar = gather_a != nullptr ? gather_a[r] : r;
          v = ld<TA>(Ap, ar * K + kx);
        }
        As[kk][mm] = v;
      }
      for (int c = tid; c < BKt * BNt; c += 256) {
        const int kk = c / BNt, nn = c % BNt;
        const int kx = k0 + kk, n = n0 + nn;
        Bs[kk][nn] = (kx < K && n < N) ? ld<TB>(Bp, static_cast<int64_t>(kx) * N + n) : 0.f;
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < BKt; ++kk) {
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
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = r0 + ty * 4 + i;
    if (r >= r1) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n < N) C[static_cast<int64_t>(r) * N + n] = acc[i][j];
    }
  }
}

// C_g[m][n] = sum over the rows r of group g of A[r][m] B[b(r)][n], b(r) = gather[r] or r;
// C is [groups][Ma][Nb]
template <typename TA, typename TB>
__global__ __launch_bounds__(256) void kk_gemm_kernel(const TA* __restrict__ A, int Ma,
                                                       const TB* __restrict__ B, int Nb,
                                                       const int32_t* __restrict__ gather,
                                                       const int32_t* __restrict__ offsets,
                                                       float* __restrict__ C) {
  __shared__ float As[BKt][BMt + 4];
  __shared__ float Bs[BKt][BNt + 4];
  const int g = blockIdx.y;
  const int nb = (Nb + BNt - 1) / BNt;
  const int m0 = static_cast<int>(blockIdx.x / nb) * BMt;
  const int n0 = static_cast<int>(blockIdx.x % nb) * BNt;
  const int rb = offsets[g], re = offsets[g + 1];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {};
  for (int k0 = rb; k0 < re; k0 += BKt) {
    for (int c = tid; c < BKt * BMt; c += 256) {
      const int kk = c / BMt, mm = c % BMt;
      const int r = k0 + kk, m = m0 + mm;
      As[kk][mm] = (r < re && m < Ma) ? ld<TA>(A, static_cast<int64_t>(r) * Ma + m) : 0.f;
    }
    for (int c = tid; c < BKt * BNt; c += 256) {
      const int kk = c / BNt, nn = c % BNt;
      const int r = k0 + kk, n = n0 + nn;
      float v = 0.f;
      if (r < re && n < Nb) {
        const int64_t br = gather != nullptr ? gather[r] : r;
        v = ld<TB>(B, br * Nb + n);
      }
      Bs[kk][nn] = v;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BKt; ++kk) {
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
  float* Cg = C + static_cast<int64_t>(g) * Ma * Nb;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= Ma) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n < Nb) Cg[static_cast<int64_t>(m) * Nb + n] = acc[i][j];
    }
  }
}

// dG = dh U SiLU'(G), dU = dh SiLU(G), elementwise over count values (G, U in the layer dtype)
template <typename T>
__global__ __launch_bounds__(256) void swiglu_bw_kernel(int64_t count, const float* __restrict__ dh,
                                                         const T* __restrict__ G,
                                                         const T* __restrict__ U,
                                                         float* __restrict__ dG,
                                                         float* __restrict__ dU) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= count) return;
  const float z = ld<T>(G, i), u = ld<T>(U, i), gh = dh[i];
  const float sg = 1.f / (1.f + expf(-z));
  dG[i] = gh * u * sg * (1.f + z * (1.f - sg));
  dU[i] = gh * z * sg;
}

// dx_t += sum_j dx_perm[row(t,j)] (slot order) + dx_sh[t]; one wave per token. With d a multiple
// of 4 lanes move float4s, 4 chunks apart per pass and all slots' loads issued before use.
__global__ __launch_bounds__(256) void bw_dx_kernel(int64_t Tn, int d, int k,
                                                     const int32_t* __restrict__ inv_perm,
                                                     const float* __restrict__ dx_perm,
                                                     const float* __restrict__ dx_sh,
                                                     float* __restrict__ dx) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= Tn) return;
  if ((d & 3) != 0) {
    for (int i = lane; i < d; i += 64) {
      float v = dx[t * d + i];
      for (int j = 0; j < k; ++j) {
        const int row = inv_perm[t * k + j];
        if (row >= 0) v += dx_perm[static_cast<int64_t>(row) * d + i];
      }
      if (dx_sh != nullptr) v += dx_sh[t * d + i];
      dx[t * d + i] = v;
    }
    return;
  }
  constexpr int U = 4, STEP = 256;
  const int my_row = lane < k ? inv_perm[t * k + lane] : -1;  // lane j: slot j's row
  for (int c0 = lane * 4; c0 < d; c0 += STEP * U) {
    float4 acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      acc[u] = c0 + u * STEP < d ? *reinterpret_cast<const float4*>(dx + t * d + c0 + u * STEP)
                                 : make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
      const int row = __builtin_amdgcn_readlane(my_row, j);
      if (row < 0) continue;
      float4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        v[u] = c0 + u * STEP < d ? *reinterpret_cast<const float4*>(
                                       dx_perm + static_cast<int64_t>(row) * d + c0 + u * STEP)
                                 : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        acc[u].x += v[u].x; acc[u].y += v[u].y; acc[u].z += v[u].z; acc[u].w += v[u].w;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * STEP;
      if (c >= d) continue;
      if (dx_sh != nullptr) {
        const float4 sv = *reinterpret_cast<const float4*>(dx_sh + t * d + c);
        acc[u].x += sv.x; acc[u].y += sv.y; acc[u].z += sv.z; acc[u].w += sv.w;
      }
      *reinterpret_cast<float4*>(dx + t * d + c) = acc[u];
    }
  }
}

// Expert choice: dx_t += the dx rows of the experts that took t, in ascending expert order
// (+ dx_sh[t]); one wave per token, the rows compacted into LDS by a ballot per 64 experts.
__global__ __launch_bounds__(256) void bw_dx_ec_kernel(int64_t Tn, int d, int E,
                                                        const int32_t* __restrict__ row_of,
                                                        const float* __restrict__ dx_perm,
                                                        const float* __restrict__ dx_sh,
                                                        float* __restrict__ dx) {
  __shared__ int lrow[4][MOE_E_MAX];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  if (t >= Tn) return;  // whole waves only: no block barrier below
  int cnt = 0;
  for (int e0 = 0; e0 < E; e0 += 64) {
    const int e = e0 + lane;
    const int row = e < E ? row_of[static_cast<int64_t>(e) * Tn + t] : -1;
    const unsigned long long m = __ballot(row >= 0);
    if (row >= 0) lrow[wave][cnt + __popcll(m & ((1ull << lane) - 1ull))] = row;
    cnt += __popcll(m);
  }
  __builtin_amdgcn_wave_barrier();
  for (int i = lane; i < d; i += 64) {
    float v = dx[t * d + i];
    for (int j = 0; j < cnt; ++j) v += dx_perm[static_cast<int64_t>(lrow[wave][j]) * d + i];
    if (dx_sh != nullptr) v += dx_sh[t * d + i];
    dx[t * d + i] = v;
  }
}

template <typename TA>
hipError_t nn_dispatch(int dtype_b, bool two, const void* A, const void* A2,
                       const int32_t* gather_a, const int32_t* offsets, const int32_t* tile_off, int groups,
                       int64_t max_tiles, const void* B, const void* B2, int64_t gstride, int N,
                       int K, float* C, hipStream_t st) {
  const int64_t grid = max_tiles * ((N + BNt - 1) / BNt);
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 gd(static_cast<unsigned>(grid)), bd(256);
  const TA* a = static_cast<const TA*>(A);
  const TA* a2 = static_cast<const TA*>(A2);
  if (dtype_b == MOE_F32) {
    const float* b = static_cast<const float*>(B);
    const float* b2 = static_cast<const float*>(B2);
    if (two)
      hipLaunchKernelGGL((nn_gemm_kernel<TA, float, true>), gd, bd, 0, st, a, a2, gather_a,
                         offsets, tile_off, groups, b, b2, gstride, N, K, C);
    else
      hipLaunchKernelGGL((nn_gemm_kernel<TA, float, false>), gd, bd, 0, st, a, a2, gather_a,
                         offsets, tile_off, groups, b, b2, gstride, N, K, C);
  } else {
    const bf16_t* b = static_cast<const bf16_t*>(B);
    const bf16_t* b2 = static_cast<const bf16_t*>(B2);
    if (two)
      hipLaunchKernelGGL((nn_gemm_kernel<TA, bf16_t, true>), gd, bd, 0, st, a, a2, gather_a,
                         offsets, tile_off, groups, b, b2, gstride, N, K, C);
    else
      hipLaunchKernelGGL((nn_gemm_kernel<TA, bf16_t, false>), gd, bd, 0, st, a, a2, gather_a,
                         offsets, tile_off, groups, b, b2, gstride, N, K, C);
  }
  return hipGetLastError();
}

template <typename TA>
hipError_t kk_dispatch(int dtype_b, const void* A, int Ma, const void* B, int Nb,
                       const int32_t* gather, const int32_t* offsets, int groups, float* C,
                       hipStream_t st) {
  const int64_t tiles = static_cast<int64_t>((Ma + BMt - 1) / BMt) * ((Nb + BNt - 1) / BNt);
  if (tiles <= 0 || groups <= 0) return hipSuccess;
  if (tiles > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 gd(static_cast<unsigned>(tiles), static_cast<unsigned>(groups)), bd(256);
  if (dtype_b == MOE_F32)
    hipLaunchKernelGGL((kk_gemm_kernel<TA, float>), gd, bd, 0, st, static_cast<const TA*>(A), Ma,
                       static_cast<const float*>(B), Nb, gather, offsets, C);
  else
    hipLaunchKernelGGL((kk_gemm_kernel<TA, bf16_t>), gd, bd, 0, st, static_cast<const TA*>(A), Ma,
                       static_cast<const bf16_t*>(B), Nb, gather, offsets, C);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bw_rows(int dtype, const int32_t* offsets, int E, int64_t R, int d, int M,
                          int k, const int32_t* perm_token, const int32_t* inv_perm,
                          const float* topk_w, const void* dy, const float* P, const float* G,
                          const float* U, float* dw, float* dG, float* dU, void* dGU, void* whp,
                          float* dout, float* wrow, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(cdiv(R, 4)));
  if (R <= 0) return hipSuccess;
  bf16_t* cat = static_cast<bf16_t*>(dGU);
  bf16_t* wh = static_cast<bf16_t*>(whp);
  if (dtype == MOE_F32) {
    const float* y = static_cast<const float*>(dy);
    if (cat != nullptr)
      hipLaunchKernelGGL((bw_rows_kernel<float, true>), grid, dim3(256), 0, st, offsets, E, d, M, k,
                         perm_token, inv_perm, topk_w, y, P, G, U, dw, dG, dU, cat, wh, dout, wrow);
    else
      hipLaunchKernelGGL((bw_rows_kernel<float, false>), grid, dim3(256), 0, st, offsets, E, d, M,
                         k, perm_token, inv_perm, topk_w, y, P, G, U, dw, dG, dU, cat, wh, dout, wrow);
  } else {
    const bf16_t* y = static_cast<const bf16_t*>(dy);
    if (cat != nullptr)
      hipLaunchKernelGGL((bw_rows_kernel<bf16_t, true>), grid, dim3(256), 0, st, offsets, E, d, M,
                         k, perm_token, inv_perm, topk_w, y, P, G, U, dw, dG, dU, cat, wh, dout, wrow);
    else
      hipLaunchKernelGGL((bw_rows_kernel<bf16_t, false>), grid, dim3(256), 0, st, offsets, E, d, M,
                         k, perm_token, inv_perm, topk_w, y, P, G, U, dw, dG, dU, cat, wh, dout, wrow);
  }
  return hipGetLastError();
}

hipError_t launch_swiglu_fwd(int64_t count, const float* G, const float* U, float* h,
                             hipStream_t st) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(swiglu_fwd_kernel, dim3(static_cast<unsigned>(cdiv(count, 256))), dim3(256),
                     0, st, count, G, U, h);
  return hipGetLastError();
}

hipError_t launch_bw_router(int64_t T, int E, int k, int renorm, int sigmoid, const float* lcol,
                            const float* scol, const int32_t* topk_idx, const int32_t* inv_perm,
                            const float* topk_w, const float* dw, const int32_t* n, double fden,
                            float lambda, float z_coef, float* dl, float* dlT, hipStream_t st) {
  hipLaunchKernelGGL(bw_router_kernel, dim3(static_cast<unsigned>(cdiv(T, 4))), dim3(256), 0, st,
                     T, E, k, renorm, sigmoid, lcol, scol, topk_idx, inv_perm, topk_w, dw, n, fden,
                     lambda, z_coef, dl, dlT);
  return hipGetLastError();
}

hipError_t launch_ec_gates(int64_t T, int E, int renorm, const int32_t* row_of,
                           const float* scol, float* wrow, hipStream_t st) {
  hipLaunchKernelGGL(ec_token_kernel<true>, dim3(static_cast<unsigned>(cdiv(T, 4))), dim3(256), 0,
                     st, T, E, renorm, 0, row_of, nullptr, scol, wrow, nullptr, nullptr, 1.0, 0.f,
                     0.f, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_bw_router_ec(int64_t T, int E, int renorm, int sigmoid, const int32_t* row_of,
                               const float* lcol, const float* scol, const float* dw,
                               const int32_t* n, double fden, float lambda, float z_coef,
                               float* dl, float* dlT, hipStream_t st) {
  hipLaunchKernelGGL(ec_token_kernel<false>, dim3(static_cast<unsigned>(cdiv(T, 4))), dim3(256),
                     0, st, T, E, renorm, sigmoid, row_of, lcol, scol, nullptr, dw, n, fden,
                     lambda, z_coef, dl, dlT);
  return hipGetLastError();
}

hipError_t launch_bw_dx_ec(int64_t T, int d, int E, const int32_t* row_of, const float* dx_perm,
                           const float* dx_sh, float* dx, hipStream_t st) {
  hipLaunchKernelGGL(bw_dx_ec_kernel, dim3(static_cast<unsigned>(cdiv(T, 4))), dim3(256), 0, st,
                     T, d, E, row_of, dx_perm, dx_sh, dx);
  return hipGetLastError();
}

hipError_t launch_nn_gemm(int dtype_a, int dtype_b, bool two, const void* A, const void* A2,
                          const int32_t* gather_a, const int32_t* offsets, const int32_t* tile_off,
                          int groups, int64_t max_tiles, const void* B, const void* B2,
                          int64_t gstride, int N, int K, float* C, hipStream_t st) {
  return dtype_a == MOE_F32
             ? nn_dispatch<float>(dtype_b, two, A, A2, gather_a, offsets, tile_off, groups,
                                  max_tiles, B, B2, gstride, N, K, C, st)
             : nn_dispatch<bf16_t>(dtype_b, two, A, A2, gather_a, offsets, tile_off, groups,
                                   max_tiles, B, B2, gstride, N, K, C, st);
}

hipError_t launch_kk_gemm(int dtype_a, int dtype_b, const void* A, int Ma, const void* B, int Nb,
                          const int32_t* gather, const int32_t* offsets, int groups, float* C,
                          hipStream_t st) {
  return dtype_a == MOE_F32
             ? kk_dispatch<float>(dtype_b, A, Ma, B, Nb, gather, offsets, groups, C, st)
             : kk_dispatch<bf16_t>(dtype_b, A, Ma, B, Nb, gather, offsets, groups, C, st);
}

hipError_t launch_swiglu_bw(int dtype, int64_t count, const float* dh, const void* G,
                            const void* U, float* dG, float* dU, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(cdiv(count, 256)));
  if (dtype == MOE_F32)
    hipLaunchKernelGGL(swiglu_bw_kernel<float>, grid, dim3(256), 0, st, count, dh,
                       static_cast<const float*>(G), static_cast<const float*>(U), dG, dU);
  else
    hipLaunchKernelGGL(swiglu_bw_kernel<bf16_t>, grid, dim3(256), 0, st, count, dh,
                       static_cast<const bf16_t*>(G), static_cast<const bf16_t*>(U), dG, dU);
  return hipGetLastError();
}

hipError_t launch_bw_dx(int64_t T, int d, int k, const int32_t* inv_perm, const float* dx_perm,
                        const float* dx_sh, float* dx, hipStream_t st) {
  hipLaunchKernelGGL(bw_dx_kernel, dim3(static_cast<unsigned>(cdiv(T, 4))), dim3(256), 0, st, T,
                     d, k, inv_perm, dx_perm, dx_sh, dx);
  return hipGetLastError();
}

}  // namespace moe

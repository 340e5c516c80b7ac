// Combine: y_t = sum_{j : inv_tj >= 0} w_tj * out_perm[inv_tj] (+ shared_t)
// ("MoE：条件计算与路由" §7 eq. (3)), the un-permute and weighted sum of the DeepseekV3MoE
// listing's last step on the adg.csdn.net notes page (§四), plus the shared-expert term.
//
// One wave per token: lane j holds slot j's row and gate, which are read out wave-uniformly; lanes
// walk the hidden dimension in 16-byte chunks, accumulate in fp32 in slot order j = 0..k-1, add the
// shared term last and round once to the output type.
//
// With balance statistics to compute (a layer forward), block 0 of either combine computes them
// (balance_stats.h) while the other blocks combine: the statistics need nothing the combine
// writes, and one block of 256 threads finishes well inside the HBM-bound combine, so they cost no
// launch of their own.
#include "balance_stats.h"

namespace moe {
namespace {

template <typename T>
struct Vec;  // one 16-byte chunk
template <>
struct Vec<bf16_t> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void load(const bf16_t* p, float* v) {
    unpack(*reinterpret_cast<const uint4*>(p), v);
  }
  __device__ __forceinline__ static void unpack(const uint4 u, float* v) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ __forceinline__ static void store(bf16_t* p, const float* v) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = static_cast<uint32_t>(f32_to_bf16(v[2 * i])) |
             (static_cast<uint32_t>(f32_to_bf16(v[2 * i + 1])) << 16);
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  }
};
template <>
struct Vec<float> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void load(const float* p, float* v) {
    const float4 u = *reinterpret_cast<const float4*>(p);
    v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
  }
  __device__ __forceinline__ static void unpack(const uint4 u, float* v) {
    v[0] = __uint_as_float(u.x); v[1] = __uint_as_float(u.y);
    v[2] = __uint_as_float(u.z); v[3] = __uint_as_float(u.w);
  }
  __device__ __forceinline__ static void store(float* p, const float* v) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};

// Per lane and pass: U chunks 64 VN elements apart; slots are taken JB at a time with every load
// of a group issued (as raw 16-byte values) before any is used, so a wave keeps JB U loads in
// flight at a modest register count.
constexpr int kU = 4, kJB = 2;

// block 0 of a combine launch that carries the statistics
__device__ __forceinline__ void stats_block(const StatsArgs& sa) {
  balance_stats<256>(sa.T, sa.E, sa.fden, sa.n, sa.gsum, sa.lse2sum, sa.hsum, sa.lambda, sa.f,
                     sa.P, sa.aux, sa.z, sa.diag, sa.b, sa.b_new, sa.gamma);
}

template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(int64_t Tn, int d, int k,
                                                       const T* __restrict__ out_perm,
                                                       const int32_t* __restrict__ inv_perm,
                                                       const float* __restrict__ topk_w,
                                                       const T* __restrict__ shared_out,
                                                       T* __restrict__ y, StatsArgs sa,
                                                       int with_stats) {
  constexpr int VN = Vec<T>::N, STEP = 64 * VN;
  if (with_stats && blockIdx.x == 0) {
    stats_block(sa);
    return;
  }
  const int lane = threadIdx.x & 63;
  const int64_t t = (static_cast<int64_t>(blockIdx.x) - with_stats) * 4 + (threadIdx.x >> 6);
  if (t >= Tn) return;
  // lane j holds slot j's row and gate; a slot's values are read out wave-uniformly
  const int my_row = lane < k ? inv_perm[t * k + lane] : -1;
  const int my_w = lane < k ? __float_as_int(topk_w[t * k + lane]) : 0;
  for (int c0 = lane * VN; c0 < d; c0 += STEP * kU) {
    float acc[kU][VN];
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int i = 0; i < VN; ++i) acc[u][i] = 0.f;
    for (int j0 = 0; j0 < k; j0 += kJB) {
      uint4 raw[kJB][kU];
      float wj[kJB];
#pragma unroll
      for (int jj = 0; jj < kJB; ++jj) {
        const int j = j0 + jj;
        const int row = j < k ? __builtin_amdgcn_readlane(my_row, j) : -1;
        wj[jj] = row >= 0 ? __int_as_float(__builtin_amdgcn_readlane(my_w, j)) : 0.f;
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int c = c0 + u * STEP;
          raw[jj][u] = (row >= 0 && c < d)
                           ? *reinterpret_cast<const uint4*>(out_perm +
                                                             static_cast<int64_t>(row) * d + c)
                           : make_uint4(0u, 0u, 0u, 0u);
        }
      }
      // slot order j = 0..k-1 (a dropped slot adds 0 * 0)
#pragma unroll
      for (int jj = 0; jj < kJB; ++jj)
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          float v[VN];
          Vec<T>::unpack(raw[jj][u], v);
#pragma unroll
          for (int i = 0; i < VN; ++i) acc[u][i] = fmaf(wj[jj], v[i], acc[u][i]);
        }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int c = c0 + u * STEP;
      if (c < d) {
        if (shared_out != nullptr) {
          float sv[VN];
          Vec<T>::load(shared_out + t * d + c, sv);
#pragma unroll
          for (int i = 0; i < VN; ++i) acc[u][i] += sv[i];
        }
        Vec<T>::store(y + t * d + c, acc[u]);
      }
    }
  }
}

// Expert-choice combine: y_t = sum over the experts e that took token t, in ascending e, of
// w_te out[row(t, e)] (+ shared_t); w_te = g_te, divided by sum of g_te' over those experts when
// renormalising. One wave per token: the lanes read the token's row and score of 64 experts at a
// time, a ballot compacts the taken ones in expert order into the wave's LDS list (and lane 0 sums
// the gates in that order), then the lanes walk the hidden dimension as in combine_kernel.
//   row_of, gcol [E][T] (row or -1; score)
template <typename T>
__global__ __launch_bounds__(256) void combine_ec_kernel(int64_t Tn, int d, int E, int renorm,
                                                          const T* __restrict__ out_perm,
                                                          const int32_t* __restrict__ row_of,
                                                          const float* __restrict__ gcol,
                                                          const T* __restrict__ shared_out,
                                                          T* __restrict__ y, StatsArgs sa,
                                                          int with_stats) {
  constexpr int VN = Vec<T>::N;
  __shared__ int lrow[4][MOE_E_MAX];
  __shared__ float lw[4][MOE_E_MAX];
  __shared__ float lden[4];
  if (with_stats && blockIdx.x == 0) {
    stats_block(sa);
    return;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = (static_cast<int64_t>(blockIdx.x) - with_stats) * 4 + wave;
  if (t >= Tn) return;  // whole waves only: no block barrier below
  int cnt = 0;
  for (int e0 = 0; e0 < E; e0 += 64) {
    const int e = e0 + lane;
    const int row = e < E ? row_of[static_cast<int64_t>(e) * Tn + t] : -1;
    const float g = e < E ? gcol[static_cast<int64_t>(e) * Tn + t] : 0.f;
    const unsigned long long m = __ballot(row >= 0);
    if (row >= 0) {
      const int pos = cnt + __popcll(m & ((1ull << lane) - 1ull));
      lrow[wave][pos] = row;
      lw[wave][pos] = g;
    }
    cnt += __popcll(m);
  }
  __builtin_amdgcn_wave_barrier();
  if (lane == 0) {
    float den = 0.f;
    for (int i = 0; i < cnt; ++i) den += lw[wave][i];
    lden[wave] = renorm && den > 0.f ? den : 1.f;
  }
  __builtin_amdgcn_wave_barrier();
  const float den = lden[wave];
  // as in combine_kernel: kJB experts and kU chunks per lane loaded before any is used
  constexpr int STEP = 64 * VN;
  for (int c0 = lane * VN; c0 < d; c0 += STEP * kU) {
    float acc[kU][VN];
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int i = 0; i < VN; ++i) acc[u][i] = 0.f;
    for (int j0 = 0; j0 < cnt; j0 += kJB) {
      uint4 raw[kJB][kU];
      float wj[kJB];
#pragma unroll
      for (int jj = 0; jj < kJB; ++jj) {
        const int j = j0 + jj;
        const int row = j < cnt ? lrow[wave][j] : -1;
        wj[jj] = row >= 0 ? lw[wave][j] / den : 0.f;
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int c = c0 + u * STEP;
          raw[jj][u] = (row >= 0 && c < d)
                           ? *reinterpret_cast<const uint4*>(out_perm +
                                                             static_cast<int64_t>(row) * d + c)
                           : make_uint4(0u, 0u, 0u, 0u);
        }
      }
      // experts in ascending order; past the token's last one nothing is added
#pragma unroll
      for (int jj = 0; jj < kJB; ++jj) {
        if (j0 + jj < cnt) {
#pragma unroll
          for (int u = 0; u < kU; ++u) {
            float v[VN];
            Vec<T>::unpack(raw[jj][u], v);
#pragma unroll
            for (int i = 0; i < VN; ++i) acc[u][i] = fmaf(wj[jj], v[i], acc[u][i]);
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int c = c0 + u * STEP;
      if (c < d) {
        if (shared_out != nullptr) {
          float v[VN];
          Vec<T>::load(shared_out + t * d + c, v);
#pragma unroll
          for (int i = 0; i < VN; ++i) acc[u][i] += v[i];
        }
        Vec<T>::store(y + t * d + c, acc[u]);
      }
    }
  }
}

}  // namespace

hipError_t launch_combine_ec(int dtype, int64_t T, int d, int E, int renorm, const void* out_perm,
                             const int32_t* row_of, const float* gcol, const void* shared_out,
                             void* y, hipStream_t st, const StatsArgs* stats) {
  const int ws = stats != nullptr ? 1 : 0;
  const StatsArgs sa = stats != nullptr ? *stats : StatsArgs{};
  const dim3 grid(static_cast<unsigned>(cdiv(T, 4) + ws));
  if (dtype == MOE_F32)
    hipLaunchKernelGGL(combine_ec_kernel<float>, grid, dim3(256), 0, st, T, d, E, renorm,
                       static_cast<const float*>(out_perm), row_of, gcol,
                       static_cast<const float*>(shared_out), static_cast<float*>(y), sa, ws);
  else
    hipLaunchKernelGGL(combine_ec_kernel<bf16_t>, grid, dim3(256), 0, st, T, d, E, renorm,
                       static_cast<const bf16_t*>(out_perm), row_of, gcol,
                       static_cast<const bf16_t*>(shared_out), static_cast<bf16_t*>(y), sa, ws);
  return hipGetLastError();
}
hipError_t launch_combine(int dtype, int64_t T, int d, int k, const void* out_perm,
                          const int32_t* inv_perm, const float* topk_w, const void* shared_out,
                          void* y, hipStream_t st, const StatsArgs* stats) {
  const int ws = stats != nullptr ? 1 : 0;
  const StatsArgs sa = stats != nullptr ? *stats : StatsArgs{};
  const dim3 grid(static_cast<unsigned>(cdiv(T, 4) + ws));
  if (dtype == MOE_F32)
    hipLaunchKernelGGL(combine_kernel<float>, grid, dim3(256), 0, st, T, d, k,
                       static_cast<const float*>(out_perm), inv_perm, topk_w,
                       static_cast<const float*>(shared_out), static_cast<float*>(y), sa, ws);
  else
    hipLaunchKernelGGL(combine_kernel<bf16_t>, grid, dim3(256), 0, st, T, d, k,
                       static_cast<const bf16_t*>(out_perm), inv_perm, topk_w,
                       static_cast<const bf16_t*>(shared_out), static_cast<bf16_t*>(y), sa, ws);
  return hipGetLastError();
}

}  // namespace moe

// Router kernel: l = x W_r^T, max-subtracted softmax with log-sum-exp, biased top-k selection,
// renormalised gates and per-block partial statistics ("MoE：条件计算与路由" §原理与演进,
// §无辅助损失负载均衡（ALF-LB）, §7 eqs. (1)-(2); "MOE大模型对比篇" §2.2 for the LSE term).
//
// One block of 256 threads (4 waves) owns kRouteTokens = 64 consecutive tokens. The logits tile
// [64 x E] never leaves the chip: bf16 inputs go through v_mfma_f32_16x16x32_bf16 with x and W_r
// k-slices staged in LDS; fp32 inputs use plain FMA loops. Each wave then walks 16 tokens: lanes
// own experts e = lane + 64 i, the softmax maximum / sum and the k argmax rounds are wave
// reductions, and equal scores go to the lower expert index. Statistics leave as per-block
// partials (expert histogram, sum of g, sum of lse^2) reduced later in a fixed order, so every
// result is bit-reproducible.
#include "moe_internal.h"

#include <math.h>

namespace moe {
namespace {

constexpr int RT = kRouteTokens;  // 64 tokens per block
constexpr int RK = 64;            // K elements staged per step
constexpr int RKP = RK + 8;       // padded LDS row (bf16 elements): 144 B keeps MFMA reads conflict-free

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct ArgMax {
  float v;
  int e;
};

__device__ __forceinline__ ArgMax better(ArgMax a, ArgMax b) {
  // larger score wins; equal scores go to the lower expert index
  return (b.v > a.v || (b.v == a.v && b.e < a.e)) ? b : a;
}

__device__ __forceinline__ ArgMax wave_argmax(ArgMax a) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    ArgMax o;
    o.v = __shfl_xor(a.v, off, 64);
    o.e = __shfl_xor(a.e, off, 64);
    a = better(a, o);
  }
  return a;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// ------------------------------------------------------------------------------------------
// Per-token routing over the logits tile in LDS, shared by both dtypes.
//   L: [RT][Ls] fp32 logits of this block's tokens.
// ------------------------------------------------------------------------------------------
__device__ void route_tokens(const float* L, int Ls, int64_t t0, int64_t T, int E, int k,
                             int renorm, const float* __restrict__ b, int32_t* __restrict__ topk_idx,
                             float* __restrict__ topk_w, int32_t* __restrict__ hist,
                             float* __restrict__ gpart, float* __restrict__ lpart, float* red) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  constexpr int EPL = MOE_E_MAX / 64;  // experts per lane, at most 4
  float gacc[EPL];
  int hcnt[EPL];
  float bias[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    gacc[i] = 0.f;
    hcnt[i] = 0;
    const int e = lane + 64 * i;
    bias[i] = (b != nullptr && e < E) ? b[e] : 0.f;
  }
  float lacc = 0.f;

  for (int tl = wave * 16; tl < wave * 16 + 16; ++tl) {
    const int64_t t = t0 + tl;
    if (t >= T) break;
    float v[EPL], g[EPL], s[EPL];
    float mloc = -INFINITY;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + 64 * i;
      v[i] = (e < E) ? L[tl * Ls + e] : -INFINITY;
      mloc = fmaxf(mloc, v[i]);
    }
    const float m = wave_max(mloc);
    float sloc = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) sloc += (lane + 64 * i < E) ? expf(v[i] - m) : 0.f;
    const float lse = m + logf(wave_sum(sloc));
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + 64 * i;
      g[i] = (e < E) ? expf(v[i] - lse) : 0.f;
      s[i] = (e < E) ? g[i] + bias[i] : -INFINITY;
      gacc[i] += g[i];
    }
    lacc += lse * lse;

    int sel[MOE_K_MAX];
    float gsel[MOE_K_MAX];
    float wsum = 0.f;
#pragma unroll
    for (int j = 0; j < MOE_K_MAX; ++j) {
      sel[j] = 0;
      gsel[j] = 0.f;
      if (j < k) {
        ArgMax a{-INFINITY, 0x7fffffff};
#pragma unroll
        for (int i = 0; i < EPL; ++i) a = better(a, ArgMax{s[i], lane + 64 * i});
        a = wave_argmax(a);
        const int owner = a.e & 63, slot = a.e >> 6;
        float gi = 0.f;
#pragma unroll
        for (int i = 0; i < EPL; ++i) gi = (slot == i) ? g[i] : gi;
        const float gs = __shfl(gi, owner, 64);
        if (lane == owner) {
#pragma unroll
          for (int i = 0; i < EPL; ++i) {
            if (slot == i) {
              s[i] = -INFINITY;
              hcnt[i] += 1;
            }
          }
        }
        sel[j] = a.e;
        gsel[j] = gs;
        wsum += gs;
      }
    }
    if (lane < k) {
      int my_e = 0;
      float my_g = 0.f;
#pragma unroll
      for (int j = 0; j < MOE_K_MAX; ++j) {
        if (lane == j) {
          my_e = sel[j];
          my_g = gsel[j];
        }
      }
      topk_idx[t * k + lane] = my_e;
      topk_w[t * k + lane] = renorm ? my_g / wsum : my_g;
    }
  }

  // block partials: sum the 4 waves in a fixed order
  float* gred = red;                          // [4][E_MAX]
  int* hred = reinterpret_cast<int*>(red + 4 * MOE_E_MAX);  // [4][E_MAX]
  float* lred = red + 8 * MOE_E_MAX;          // [4]
  __syncthreads();
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    gred[wave * MOE_E_MAX + e] = gacc[i];
    hred[wave * MOE_E_MAX + e] = hcnt[i];
  }
  if (lane == 0) lred[wave] = lacc;
  __syncthreads();
  const int64_t blk = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    float gs = gred[e];
    int hs = hred[e];
    for (int w = 1; w < 4; ++w) {
      gs += gred[w * MOE_E_MAX + e];
      hs += hred[w * MOE_E_MAX + e];
    }
    gpart[blk * E + e] = gs;
    hist[blk * E + e] = hs;
  }
  if (threadIdx.x == 0) lpart[blk] = ((lred[0] + lred[1]) + lred[2]) + lred[3];
}

// LDS budget: max(logits tile, staged k-slices) plus the reduction scratch.
constexpr int kLogitsStride = MOE_E_MAX + 4;
constexpr int kTileBytes = (RT + MOE_E_MAX) * RKP * 2;
constexpr int kLogitsBytes = RT * kLogitsStride * 4;
constexpr int kUnionBytes = kTileBytes > kLogitsBytes ? kTileBytes : kLogitsBytes;
constexpr int kRedFloats = 8 * MOE_E_MAX + 4;

// ------------------------------------------------------------------------------------------
// bf16: logits on MFMA. Wave w computes tokens [16w, 16w+16) against all NEB expert blocks of 16.
// Fragment layout of v_mfma_f32_16x16x32_bf16: lane l supplies row (l % 16) of A and column
// (l % 16) of B with 8 consecutive k values of k-group (l / 16); the result element
// (row 4*(l/16) + j, column l % 16) lands in lane l, register j.
// ------------------------------------------------------------------------------------------
template <int NEB>
__global__ __launch_bounds__(256) void route_bf16_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ W, const float* __restrict__ b,
    int64_t T, int d, int E, int k, int renorm, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, int32_t* __restrict__ hist, float* __restrict__ gpart,
    float* __restrict__ lpart) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kUnionBytes];
  __shared__ float red[kRedFloats];
  bf16_t* xs = reinterpret_cast<bf16_t*>(smem);  // [RT][RKP]
  bf16_t* ws = xs + RT * RKP;                    // [NEB*16][RKP]
  constexpr int ER = NEB * 16;                   // padded expert rows
  constexpr int XCH = RT * (RK / 8);             // 16-byte chunks of the x slice (512)
  constexpr int WCH = ER * (RK / 8);             // 16-byte chunks of the W_r slice
  constexpr int XPT = XCH / 256;                 // per thread (2)
  constexpr int WPT = (WCH + 255) / 256;         // per thread (<= 8)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * RT;

  uint4 xr[XPT], wr[WPT];
  auto load_slices = [&](int k0) {
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int c = i * 256 + tid, row = c >> 3, col = (c & 7) * 8;
      int64_t t = t0 + row;
      t = t < T ? t : T - 1;
      xr[i] = (k0 + col < d) ? *reinterpret_cast<const uint4*>(x + t * d + k0 + col)
                             : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      const int c = i * 256 + tid, row = c >> 3, col = (c & 7) * 8;
      wr[i] = (c < WCH && row < E && k0 + col < d)
                  ? *reinterpret_cast<const uint4*>(W + static_cast<int64_t>(row) * d + k0 + col)
                  : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_slices = [&]() {
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int c = i * 256 + tid, row = c >> 3, col = (c & 7) * 8;
      *reinterpret_cast<uint4*>(xs + row * RKP + col) = xr[i];
    }
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      const int c = i * 256 + tid, row = c >> 3, col = (c & 7) * 8;
      if (c < WCH) *reinterpret_cast<uint4*>(ws + row * RKP + col) = wr[i];
    }
  };

  f32x4 acc[NEB];
#pragma unroll
  for (int j = 0; j < NEB; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int r16 = lane & 15, kg = lane >> 4;
  load_slices(0);
  for (int k0 = 0; k0 < d; k0 += RK) {
    __syncthreads();  // previous step's LDS reads are done
    store_slices();
    __syncthreads();
    if (k0 + RK < d) load_slices(k0 + RK);  // next slice in flight during the MFMAs
#pragma unroll
    for (int sub = 0; sub < RK / 32; ++sub) {
      const int kc = sub * 32 + kg * 8;
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(xs + (wave * 16 + r16) * RKP + kc);
#pragma unroll
      for (int j = 0; j < NEB; ++j) {
        const bf16x8 bb = *reinterpret_cast<const bf16x8*>(ws + (j * 16 + r16) * RKP + kc);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bb, acc[j], 0, 0, 0);
      }
    }
  }
  __syncthreads();
  float* L = reinterpret_cast<float*>(smem);  // [RT][kLogitsStride], reuses the slice buffers
#pragma unroll
  for (int j = 0; j < NEB; ++j) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = wave * 16 + kg * 4 + r, col = j * 16 + r16;
      L[row * kLogitsStride + col] = acc[j][r];
    }
  }
  __syncthreads();
  route_tokens(L, kLogitsStride, t0, T, E, k, renorm, b, topk_idx, topk_w, hist, gpart, lpart, red);
}

// ------------------------------------------------------------------------------------------
// fp32: logits by sequential FMA over the hidden dimension (one (token, expert) pair per thread).
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void route_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ W, const float* __restrict__ b,
    int64_t T, int d, int E, int k, int renorm, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, int32_t* __restrict__ hist, float* __restrict__ gpart,
    float* __restrict__ lpart) {
  __shared__ float L[RT * kLogitsStride];
  __shared__ float red[kRedFloats];
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * RT;
  for (int p = threadIdx.x; p < RT * E; p += blockDim.x) {
    const int tl = p / E, e = p % E;
    int64_t t = t0 + tl;
    t = t < T ? t : T - 1;
    const float* xr = x + t * d;
    const float* wr = W + static_cast<int64_t>(e) * d;
    float acc = 0.f;
    for (int i = 0; i < d; ++i) acc = fmaf(xr[i], wr[i], acc);
    L[tl * kLogitsStride + e] = acc;
  }
  __syncthreads();
  route_tokens(L, kLogitsStride, t0, T, E, k, renorm, b, topk_idx, topk_w, hist, gpart, lpart, red);
}

template <int NEB>
hipError_t launch_bf16(int64_t nblk, hipStream_t st, const void* x, const void* W, const float* b,
                       int64_t T, int d, int E, int k, int renorm, int32_t* topk_idx,
                       float* topk_w, int32_t* hist, float* gpart, float* lpart) {
  hipLaunchKernelGGL(route_bf16_kernel<NEB>, dim3(static_cast<unsigned>(nblk)), dim3(256), 0, st,
                     static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(W), b, T, d, E, k,
                     renorm, topk_idx, topk_w, hist, gpart, lpart);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(int dtype, int64_t T, int d, int E, int k, int renorm, const void* x,
                        const void* W_r, const float* b, int32_t* topk_idx, float* topk_w,
                        int32_t* hist, float* gpart, float* lpart, hipStream_t st) {
  const int64_t nblk = cdiv(T, RT);
  if (dtype == MOE_F32) {
    hipLaunchKernelGGL(route_f32_kernel, dim3(static_cast<unsigned>(nblk)), dim3(256), 0, st,
                       static_cast<const float*>(x), static_cast<const float*>(W_r), b, T, d, E,
                       k, renorm, topk_idx, topk_w, hist, gpart, lpart);
    return hipGetLastError();
  }
  const int neb = static_cast<int>(cdiv(E, 16));
#define MOE_ROUTE_CASE(N) \
  case N:                 \
    return launch_bf16<N>(nblk, st, x, W_r, b, T, d, E, k, renorm, topk_idx, topk_w, hist, gpart, lpart);
  switch (neb) {
    MOE_ROUTE_CASE(1) MOE_ROUTE_CASE(2) MOE_ROUTE_CASE(3) MOE_ROUTE_CASE(4)
    MOE_ROUTE_CASE(5) MOE_ROUTE_CASE(6) MOE_ROUTE_CASE(7) MOE_ROUTE_CASE(8)
    MOE_ROUTE_CASE(9) MOE_ROUTE_CASE(10) MOE_ROUTE_CASE(11) MOE_ROUTE_CASE(12)
    MOE_ROUTE_CASE(13) MOE_ROUTE_CASE(14) MOE_ROUTE_CASE(15) MOE_ROUTE_CASE(16)
    default:
      return hipErrorInvalidValue;
  }
#undef MOE_ROUTE_CASE
}

}  // namespace moe

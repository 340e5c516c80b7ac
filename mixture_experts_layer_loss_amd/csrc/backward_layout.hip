// Operand layouts for the bf16 backward products on MFMA. The products that reduce over d or M
// against a weight (P = dy W_down[e], dx_row = dG W_gate[e] + dU W_up[e]) read the weights in place
// (the grouped GEMM's K-major B path); the weight gradients reduce over rows, so the backward feeds
// them transposed copies:
//   - the row operands of the weight gradients, with the rows of each expert as columns, each
//     expert's column range padded with zeros to a multiple of 64: the gathered dy^T, (w h)^T,
//     dG^T, dU^T and the gathered x^T (dW_down[e] = sum over its rows of dy_t^T (w h), dW_gate[e] =
//     dG_e^T x_e, dW_up[e] = dU_e^T x_e). Every product thus has one operand that was rounded to
//     bf16 here (w h, dG, dU) and one exact bf16 input (dy, x, the weights).
// The SwiGLU derivative ("深入理解 MoE (混合专家模型)：稀疏激活与高效扩展" §10.2) is written here as
// one bf16 row [dG | dU] per kept row, the A operand of the dx product. The transposes keep both
// their reads and their writes in contiguous runs of 128 bytes or more.
#include "moe_internal.h"

#include <math.h>

namespace moe {
namespace {

constexpr int TT = 64;       // tile edge
constexpr int TP = TT + 2;   // LDS row pitch (elements)

template <typename T>
__device__ __forceinline__ void load8(const T* p, float* v);
template <>
__device__ __forceinline__ void load8<float>(const float* p, float* v) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
template <>
__device__ __forceinline__ void load8<bf16_t>(const bf16_t* p, float* v) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// dst [cols][ldp] bf16: column p of group g (p in [64 kt[g], 64 kt[g+1])) holds source row
// i = off[g] + p - 64 kt[g] (row gather[i] of src when gather != NULL; src rows ld_src apart),
// times scale[i] when scale != NULL, or zeros past the group's rows; rounded once to bf16. SWI: the
// source value is SiLU(src) src2 (fp32 pre-activations G, U). cols a multiple of 8. Tiles past
// 64 kt[groups] are left alone.
template <typename TS, bool SWI>
__global__ __launch_bounds__(256) void pad_transpose_kernel(
    const TS* __restrict__ src, const float* __restrict__ src2, int64_t ld_src,
    const int32_t* __restrict__ gather,
    const float* __restrict__ scale, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ kt, int groups, int cols, bf16_t* __restrict__ dst,
    int64_t ldp) {
  __shared__ uint16_t tile[TT][TP];  // [p][c]
  const int tid = threadIdx.x;
  const int pt = blockIdx.x, c0 = blockIdx.y * TT;
  if (pt >= kt[groups]) return;
  int lo = 0, hi = groups;  // largest g with kt[g] <= pt (a group owning no tile is skipped)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (kt[mid] <= pt) lo = mid; else hi = mid;
  }
  const int g = lo;
  const int row0 = offsets[g] + (pt - kt[g]) * TT, row_end = offsets[g + 1];
  const int cc = (tid & 7) * 8;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int p = (tid >> 3) + pass * 32;
    const int row = row0 + p;
    float v[8];
    if (row < row_end && c0 + cc < cols) {
      const int64_t sr = gather != nullptr ? gather[row] : row;
      load8<TS>(src + sr * ld_src + c0 + cc, v);
      if constexpr (SWI) {
        float u[8];
        load8<float>(src2 + sr * ld_src + c0 + cc, u);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = v[i] / (1.f + expf(-v[i])) * u[i];
      }
      if (scale != nullptr) {
        const float sc = scale[row];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] *= sc;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) tile[p][cc + i] = f32_to_bf16(v[i]);
  }
  __syncthreads();
  const int pp = (tid & 7) * 8;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int c = (tid >> 3) + pass * 32;
    if (c0 + c < cols) {
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = static_cast<uint32_t>(tile[pp + 2 * i][c]) |
               (static_cast<uint32_t>(tile[pp + 2 * i + 1][c]) << 16);
      *reinterpret_cast<uint4*>(dst + static_cast<int64_t>(c0 + c) * ldp +
                                static_cast<int64_t>(pt) * TT + pp) =
          make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// dGU[r] = [dh U SiLU'(G) | dh SiLU(G)] (bf16, 2M per row) from fp32 dh, G, U [R][M]
__global__ __launch_bounds__(256) void swiglu_bw_cat_kernel(int64_t count, int M,
                                                             const float* __restrict__ dh,
                                                             const float* __restrict__ G,
                                                             const float* __restrict__ U,
                                                             bf16_t* __restrict__ dGU) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= count) return;
  const int64_t r = i / M, m = i - r * M;
  const float z = G[i], u = U[i], gh = dh[i];
  const float sg = 1.f / (1.f + expf(-z));
  dGU[r * 2 * M + m] = f32_to_bf16(gh * u * sg * (1.f + z * (1.f - sg)));
  dGU[r * 2 * M + M + m] = f32_to_bf16(gh * z * sg);
}

}  // namespace

hipError_t launch_pad_transpose(int dtype_src, const void* src, const float* src2, int64_t ld_src,
                                const int32_t* gather, const float* scale,
                                const int32_t* offsets, const int32_t* kt, int groups,
                                int64_t max_ptiles, int cols, void* dst, int64_t ldp,
                                hipStream_t st) {
  if (max_ptiles <= 0 || cols <= 0) return hipSuccess;
  if (src2 != nullptr && dtype_src != MOE_F32) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(max_ptiles), static_cast<unsigned>(cdiv(cols, TT)));
  bf16_t* o = static_cast<bf16_t*>(dst);
  if (src2 != nullptr)
    hipLaunchKernelGGL((pad_transpose_kernel<float, true>), grid, dim3(256), 0, st,
                       static_cast<const float*>(src), src2, ld_src, gather, scale, offsets, kt,
                       groups, cols, o, ldp);
  else if (dtype_src == MOE_F32)
    hipLaunchKernelGGL((pad_transpose_kernel<float, false>), grid, dim3(256), 0, st,
                       static_cast<const float*>(src), nullptr, ld_src, gather, scale, offsets, kt,
                       groups, cols, o, ldp);
  else
    hipLaunchKernelGGL((pad_transpose_kernel<bf16_t, false>), grid, dim3(256), 0, st,
                       static_cast<const bf16_t*>(src), nullptr, ld_src, gather, scale, offsets,
                       kt, groups, cols, o, ldp);
  return hipGetLastError();
}

hipError_t launch_swiglu_bw_cat(int64_t R, int M, const float* dh, const float* G, const float* U,
                                void* dGU, hipStream_t st) {
  const int64_t count = R * M;
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(swiglu_bw_cat_kernel, dim3(static_cast<unsigned>(cdiv(count, 256))),
                     dim3(256), 0, st, count, M, dh, G, U, static_cast<bf16_t*>(dGU));
  return hipGetLastError();
}

}  // namespace moe

// Operand layouts for the bf16 backward products on MFMA. The products that reduce over d or M
// against a weight (P = dy W_down[e], dx_row = dG W_gate[e] + dU W_up[e]) read the weights in place
// (the grouped GEMM's K-major B path); the weight gradients reduce over rows and read their row
// operands in place too, K-major: dW_down[e] = sum over its rows of dy_t^T (w h), dW_gate[e] =
// dG_e^T x_e, dW_up[e] = dU_e^T x_e. This file writes the rows they read in routed order: the
// gathered dy and x rows, and for the shared experts h; bw_rows writes w h. Every product thus has
// one operand that was rounded to bf16 (w h, h, dG, dU) and one exact bf16 input (dy, x, a weight).
// The SwiGLU derivative ("深入理解 MoE (混合专家模型)：稀疏激活与高效扩展" §10.2) is written as one
// bf16 row [dG | dU] per row, the A operand of the dx product.
#include "moe_internal.h"

#include <math.h>

namespace moe {
namespace {

// dst[r] = src[gather[r]] for the kept rows r < offsets[groups]: one wave per row, 16-byte chunks
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint4* __restrict__ src,
                                                          int chunks, const int32_t* __restrict__ gather,
                                                          const int32_t* __restrict__ offsets,
                                                          int groups, uint4* __restrict__ dst) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (r >= offsets[groups]) return;
  const int64_t t = gather[r];
  for (int c = threadIdx.x & 63; c < chunks; c += 64) dst[r * chunks + c] = src[t * chunks + c];
}

// dGU[r] = [dh U SiLU'(G) | dh SiLU(G)] (bf16, 2M per row) and h[r] = SiLU(G) U (bf16, M per
// row) from fp32 dh, G, U [R][M]
__global__ __launch_bounds__(256) void swiglu_bw_cat_kernel(int64_t count, int M,
                                                             const float* __restrict__ dh,
                                                             const float* __restrict__ G,
                                                             const float* __restrict__ U,
                                                             bf16_t* __restrict__ dGU,
                                                             bf16_t* __restrict__ h) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= count) return;
  const int64_t r = i / M, m = i - r * M;
  const float z = G[i], u = U[i], gh = dh[i];
  const float sg = 1.f / (1.f + expf(-z));
  dGU[r * 2 * M + m] = f32_to_bf16(gh * u * sg * (1.f + z * (1.f - sg)));
  dGU[r * 2 * M + M + m] = f32_to_bf16(gh * z * sg);
  h[i] = f32_to_bf16(z / (1.f + expf(-z)) * u);
}

}  // namespace

hipError_t launch_gather_rows(const void* src, int d, const int32_t* gather,
                              const int32_t* offsets, int groups, int64_t R, void* dst,
                              hipStream_t st) {
  if (R <= 0) return hipSuccess;
  if (d % 8 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gather_rows_kernel, dim3(static_cast<unsigned>(cdiv(R, 4))), dim3(256), 0, st,
                     static_cast<const uint4*>(src), d / 8, gather, offsets, groups,
                     static_cast<uint4*>(dst));
  return hipGetLastError();
}

hipError_t launch_swiglu_bw_cat(int64_t R, int M, const float* dh, const float* G, const float* U,
                                void* dGU, void* h, hipStream_t st) {
  const int64_t count = R * M;
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(swiglu_bw_cat_kernel, dim3(static_cast<unsigned>(cdiv(count, 256))),
                     dim3(256), 0, st, count, M, dh, G, U, static_cast<bf16_t*>(dGU),
                     static_cast<bf16_t*>(h));
  return hipGetLastError();
}

}  // namespace moe

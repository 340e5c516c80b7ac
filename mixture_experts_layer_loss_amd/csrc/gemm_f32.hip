// Grouped SwiGLU experts in fp32 ("深入理解 MoE (混合专家模型)：稀疏激活与高效扩展" §10.2) for
// the fp32 layer. 64 x 64 output tiles, 256 threads, 4 x 4 outputs per thread, K staged 16 at a
// time in LDS; the SwiGLU variant accumulates gate and up side by side. The fp32 layer is a
// correctness workload of a few MFLOP, so this path favours simplicity over peak throughput.
#include "moe_internal.h"

#include <math.h>

namespace moe {
namespace {

constexpr int BM = kGemmF32BM;  // 64
constexpr int BN = 64;
constexpr int BK = 16;

// EPI 0: SwiGLU (B0 = W_gate, B1 = W_up), 1: plain (B0 = W_down). gather (may be NULL): A row r
// is A[gather[r]].
template <int EPI>
__global__ __launch_bounds__(256) void grouped_gemm_f32_kernel(
    const float* __restrict__ A, const int32_t* __restrict__ gather,
    const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ tile_off, int groups, const float* __restrict__ B0,
    const float* __restrict__ B1, int64_t group_stride, int N, int K, float* __restrict__ C) {
  __shared__ float As[BK][BM + 1];
  __shared__ float Bs[2][BK][BN + 1];
  const int nb_count = (N + BN - 1) / BN;
  const int64_t ntiles = static_cast<int64_t>(tile_off[groups]) * nb_count;
  const int64_t L = blockIdx.x;
  if (L >= ntiles) return;
  int lo = 0, hi = groups;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (static_cast<int64_t>(tile_off[mid]) * nb_count <= L) lo = mid; else hi = mid;
  }
  const int g = lo;
  const int mt_g = tile_off[g + 1] - tile_off[g];
  const int64_t local = L - static_cast<int64_t>(tile_off[g]) * nb_count;
  const int n0 = static_cast<int>(local / mt_g) * BN;
  const int row_begin = offsets[g] + static_cast<int>(local % mt_g) * BM;
  const int row_end = min(row_begin + BM, offsets[g + 1]);
  const float* Bg[2] = {B0 + static_cast<int64_t>(g) * group_stride,
                        EPI == 0 ? B1 + static_cast<int64_t>(g) * group_stride : nullptr};

  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  float acc[2][4][4] = {};
  for (int k0 = 0; k0 < K; k0 += BK) {
    for (int c = tid; c < BM * BK; c += 256) {
      const int r = c / BK, kk = c % BK;
      int ar = min(row_begin + r, row_end - 1);
      if (gather != nullptr) ar = gather[ar];
      As[kk][r] = (k0 + kk < K) ? A[static_cast<int64_t>(ar) * K + k0 + kk] : 0.f;
#pragma unroll
      for (int m = 0; m < (EPI == 0 ? 2 : 1); ++m) {
        const int br = min(n0 + r, N - 1);
        Bs[m][kk][r] = (k0 + kk < K) ? Bg[m][static_cast<int64_t>(br) * K + k0 + kk] : 0.f;
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float a[4], bv[2][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int m = 0; m < (EPI == 0 ? 2 : 1); ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j) bv[m][j] = Bs[m][kk][tx * 4 + j];
#pragma unroll
      for (int m = 0; m < (EPI == 0 ? 2 : 1); ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[m][i][j] = fmaf(a[i], bv[m][j], acc[m][i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = row_begin + ty * 4 + i;
    if (r >= row_end) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= N) continue;
      float v = acc[0][i][j];
      if (EPI == 0) v = v / (1.0f + expf(-v)) * acc[1][i][j];
      C[static_cast<int64_t>(r) * N + n] = v;
    }
  }
}

}  // namespace

hipError_t launch_gemm_up_f32(int groups, int d, int Mg, const void* rows,
                              const int32_t* gather, const int32_t* offsets,
                              const int32_t* tile_off, int64_t max_tiles, const void* W_gate,
                              const void* W_up, void* h, hipStream_t st) {
  const int64_t grid = max_tiles * cdiv(Mg, BN);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(grouped_gemm_f32_kernel<0>, dim3(static_cast<unsigned>(grid)), dim3(256), 0,
                     st, static_cast<const float*>(rows), gather, offsets, tile_off, groups,
                     static_cast<const float*>(W_gate), static_cast<const float*>(W_up),
                     static_cast<int64_t>(Mg) * d, Mg, d, static_cast<float*>(h));
  return hipGetLastError();
}

hipError_t launch_gemm_plain_f32(int groups, const void* rows, const int32_t* gather,
                                 const int32_t* offsets, const int32_t* tile_off,
                                 int64_t max_tiles, const void* B, int64_t group_stride, int N,
                                 int K, void* C, hipStream_t st) {
  const int64_t grid = max_tiles * cdiv(N, BN);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(grouped_gemm_f32_kernel<1>, dim3(static_cast<unsigned>(grid)), dim3(256), 0,
                     st, static_cast<const float*>(rows), gather, offsets, tile_off, groups,
                     static_cast<const float*>(B), nullptr, group_stride, N, K,
                     static_cast<float*>(C));
  return hipGetLastError();
}

hipError_t launch_gemm_down_f32(int groups, int d, int Mg, const int32_t* offsets,
                                const int32_t* tile_off, int64_t max_tiles, const void* W_down,
                                const void* h, void* out, hipStream_t st) {
  const int64_t grid = max_tiles * cdiv(d, BN);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(grouped_gemm_f32_kernel<1>, dim3(static_cast<unsigned>(grid)), dim3(256), 0,
                     st, static_cast<const float*>(h), nullptr, offsets, tile_off, groups,
                     static_cast<const float*>(W_down), nullptr, static_cast<int64_t>(Mg) * d, d,
                     Mg, static_cast<float*>(out));
  return hipGetLastError();
}

}  // namespace moe

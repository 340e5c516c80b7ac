// Grouped expert GEMMs on bf16 MFMA for gfx950 (the SwiGLU experts of "深入理解 MoE (混合专家模型)：
// 稀疏激活与高效扩展" §10.2: h = SiLU(X W_1^T) ⊙ (X W_3^T), out = h W_2^T).
//
// Both products are "TN": every operand row is contiguous along the reduction dimension K, so A
// rows and B rows are read with 16-byte vector loads. A block of 256 threads (4 waves, 2 x 2)
// computes a 256 x 256 tile with v_mfma_f32_32x32x16_bf16; each wave owns 128 x 128 (16 MFMA
// blocks, 256 fp32 accumulators per lane). K advances 64 at a time through two LDS stages of
// 64 KiB (A and B slices, XOR-swizzled 16-byte chunks so the MFMA fragment reads and the stores
// are bank-conflict-free) with the next slice prefetched into registers during the MFMAs.
//
// Gate/up fusion: the B tile's first 128 rows come from W_gate and the last 128 from W_up at the
// same output columns, so a lane holds gate and up values of the same (row, column) and applies
// SiLU(g) * u in registers; h leaves as bf16. The down projection uses 256 plain columns.
//
// Groups (experts) are ragged: the tile table tile_off[g] (exclusive prefix of ceil(rows_g/256))
// lives on the device, the grid is an upper bound, and each block finds its (group, n-block,
// m-tile) from its logical index. Logical tiles are ordered group-major, then n-block, with the
// m-tiles of a group fastest, and consecutive logical tiles are kept on one XCD (blocks are dealt
// to the 8 XCDs round-robin), so the blocks sharing a weight slice or a row slice share an L2.
#include "moe_internal.h"

#include <math.h>

#include <atomic>
#include <type_traits>

namespace moe {
namespace {

constexpr int BM = kGemmBM;  // 256
constexpr int BN = 256;      // B rows per tile
constexpr int BK = 64;
constexpr int NXCD = 8;
constexpr int kStageElems = (BM + BN) * BK;  // bf16 elements per LDS stage (64 KiB)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // native 16-byte value (no struct copy)
typedef float f32x16 __attribute__((ext_vector_type(16)));

// element offset of 16-byte chunk `c` (0..7) of row `r` in a [rows][64] swizzled slice
__device__ __forceinline__ int swz(int r, int c) { return r * BK + ((c ^ ((r >> 1) & 7)) << 3); }

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// Instruction-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSgMfma = 0x008, kSgVmemRead = 0x020, kSgDsRead = 0x100, kSgDsWrite = 0x200;

// Schedule of one sub-step: one MFMA then one fragment read (x8), then 8 MFMAs each followed by
// EXTRA_PER instructions of group EXTRA_MASK (LDS stores or global loads), if any.
template <int EXTRA_MASK, int EXTRA_PER>
__device__ __forceinline__ void sched_substep() {
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
    if (EXTRA_PER > 0) __builtin_amdgcn_sched_group_barrier(EXTRA_MASK, EXTRA_PER, 0);
  }
}

// EPI 0: SwiGLU (B0 = W_gate, B1 = W_up, 128 output columns per tile); EPI 1: plain (B0 = W_down).
// KTAIL: K is not a multiple of 64 (the last k-slice is zero-padded).
template <int EPI, bool KTAIL>
__global__ __launch_bounds__(256, 1) void grouped_gemm_kernel(
    const bf16_t* __restrict__ A, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ tile_off, int groups, const bf16_t* __restrict__ B0,
    const bf16_t* __restrict__ B1, int64_t group_stride, int N, int K, bf16_t* __restrict__ C) {
  constexpr int BNO = EPI == 0 ? BN / 2 : BN;  // output columns per tile
  extern __shared__ __attribute__((aligned(16))) bf16_t smem[];

  // ---- which tile: XCD-contiguous logical index, then (group, n-block, m-tile)
  const int nb_count = (N + BNO - 1) / BNO;
  const int64_t ntiles = static_cast<int64_t>(tile_off[groups]) * nb_count;
  const int64_t q = (ntiles + NXCD - 1) / NXCD;
  const int64_t L = static_cast<int64_t>(blockIdx.x % NXCD) * q + blockIdx.x / NXCD;
  if (blockIdx.x / NXCD >= q || L >= ntiles) return;
  int lo = 0, hi = groups;  // largest g with tile_off[g] * nb_count <= L
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (static_cast<int64_t>(tile_off[mid]) * nb_count <= L) lo = mid; else hi = mid;
  }
  const int g = lo;
  const int mt_g = tile_off[g + 1] - tile_off[g];
  const int64_t local = L - static_cast<int64_t>(tile_off[g]) * nb_count;
  const int nb = static_cast<int>(local / mt_g);
  const int mt = static_cast<int>(local % mt_g);
  const int row_begin = offsets[g] + mt * BM;
  const int row_end = min(offsets[g] + (mt + 1) * BM, offsets[g + 1]);
  const int n0 = nb * BNO;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int rows_here = row_end - row_begin;
  unsigned char* lds = reinterpret_cast<unsigned char*>(smem);

  // ---- global loads: thread `tid` moves chunk (tid & 7) of rows r0 + 32 i (i = 0..7) of the A and
  // B k-slices. Addresses are uniform tile bases plus 32-bit byte offsets fixed over K; rows past
  // the group (A) or past N (B) re-read the last valid row and never reach a stored output.
  const int r0 = tid >> 3, kc_t = (tid & 7) * 8;
  const char* a_base = reinterpret_cast<const char*>(A + static_cast<int64_t>(row_begin) * K);
  const bf16_t* Bg0 = B0 + static_cast<int64_t>(g) * group_stride + static_cast<int64_t>(n0) * K;
  const bf16_t* Bg1 =
      EPI == 0 ? B1 + static_cast<int64_t>(g) * group_stride + static_cast<int64_t>(n0) * K : Bg0;
  const char* b_base0 = reinterpret_cast<const char*>(Bg0);
  const char* b_base1 = reinterpret_cast<const char*>(Bg1);
  const int b_rows = min(EPI == 0 ? BN / 2 : BN, N - n0);
  uint32_t a_off[8], b_off[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = i * 32 + r0;
    a_off[i] = static_cast<uint32_t>((min(r, rows_here - 1) * K + kc_t) * 2);
    const int rb_ = EPI == 0 ? (r & (BN / 2 - 1)) : r;
    b_off[i] = static_cast<uint32_t>((min(rb_, b_rows - 1) * K + kc_t) * 2);
  }
  u32x4 ra[8], rb[8];
  auto gload = [&](int k0) __attribute__((always_inline)) {
    if (KTAIL) {
      // a chunk past K re-reads the row's last chunk and is then zeroed
      const bool in = k0 + kc_t < K;
      const uint32_t kb = static_cast<uint32_t>((in ? k0 : K - 8 - kc_t) * 2);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const char* bb = (EPI == 0 && i >= 4) ? b_base1 : b_base0;
        const u32x4 va = *reinterpret_cast<const u32x4*>(a_base + (a_off[i] + kb));
        const u32x4 vb = *reinterpret_cast<const u32x4*>(bb + (b_off[i] + kb));
        const u32x4 zero = {0u, 0u, 0u, 0u};
        ra[i] = in ? va : zero;
        rb[i] = in ? vb : zero;
      }
    } else {
      const uint32_t kb = static_cast<uint32_t>(k0 * 2);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const char* bb = (EPI == 0 && i >= 4) ? b_base1 : b_base0;
        ra[i] = *reinterpret_cast<const u32x4*>(a_base + (a_off[i] + kb));
        rb[i] = *reinterpret_cast<const u32x4*>(bb + (b_off[i] + kb));
      }
    }
  };
  // LDS byte offset of this thread's chunk of row r0; row r0 + 32 i sits 32 * 128 B further on
  // (the swizzle term depends on (r >> 1) & 7, which is the same for all i)
  const uint32_t st_off = static_cast<uint32_t>(swz(r0, tid & 7) * 2);
  constexpr uint32_t kStageBytes = kStageElems * 2, kBBytes = BM * BK * 2;
  auto lstore = [&](int stage) __attribute__((always_inline)) {
    unsigned char* sa = lds + stage * kStageBytes + st_off;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      *reinterpret_cast<u32x4*>(sa + i * 32 * BK * 2) = ra[i];
      *reinterpret_cast<u32x4*>(sa + kBBytes + i * 32 * BK * 2) = rb[i];
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // ---- MFMA fragments: lane l reads row (l % 32) of a 32-row block, k-chunk 2*sub + l/32.
  // Every block starts at a multiple of 32 rows, so the swizzle term is the lane's own.
  const int l32 = lane & 31, lk = lane >> 5, sw = (l32 >> 1) & 7;
  uint32_t fo[4];
#pragma unroll
  for (int sub = 0; sub < 4; ++sub)
    fo[sub] = static_cast<uint32_t>((l32 * BK + (((sub * 2 + lk) ^ sw) << 3)) * 2);
  int brow[4];  // B-tile rows of this wave's four 32-column blocks
#pragma unroll
  for (int j = 0; j < 4; ++j)
    brow[j] = EPI == 0 ? ((j < 2 ? 0 : BN / 2) + wn * 64 + (j & 1) * 32) : (wn * 128 + j * 32);
  bf16x8 fa[2][4], fb[2][4];
  auto lfrag = [&](int set, int stage, int sub) __attribute__((always_inline)) {
    const unsigned char* sa = lds + stage * kStageBytes + fo[sub];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      fa[set][i] = *reinterpret_cast<const bf16x8*>(sa + (wm * 128 + i * 32) * BK * 2);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      fb[set][j] = *reinterpret_cast<const bf16x8*>(sa + kBBytes + brow[j] * BK * 2);
  };
  auto mfmas = [&](int set) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[set][i], fb[set][j], acc[i][j], 0, 0, 0);
  };
  // ---- main loop. A k-step (64 of K) is 4 sub-steps of 16 MFMAs on stage `cur`:
  //   sub 0: read fragments of sub 1                    | MFMAs of sub 0
  //   sub 1: read fragments of sub 2, store stage cur^1 | MFMAs of sub 1
  //   sub 2: read fragments of sub 3, load k-step +2    | MFMAs of sub 2
  //   barrier (stage cur^1 complete; every read of stage cur issued)
  //   sub 3: read fragments of sub 0 of stage cur^1     | MFMAs of sub 3
  // Global loads run ~1.5 k-steps ahead; no LDS read waits on a barrier.
  auto kstep = [&](int kt, auto has_next, auto has_load) __attribute__((always_inline)) {
    constexpr bool NEXT = decltype(has_next)::value;  // a following k-step exists
    constexpr bool LOAD = decltype(has_load)::value;  // k-step kt + 2 exists
    const int cur = kt & 1;
    lfrag(1, cur, 1);
    mfmas(0);
    sched_substep<0, 0>();
    lfrag(0, cur, 2);
    mfmas(1);
    if constexpr (NEXT) {
      lstore(cur ^ 1);
      sched_substep<kSgDsWrite, 2>();
    } else {
      sched_substep<0, 0>();
    }
    lfrag(1, cur, 3);
    mfmas(0);
    if constexpr (LOAD) {
      gload((kt + 2) * BK);
      sched_substep<kSgVmemRead, 2>();
    } else {
      sched_substep<0, 0>();
    }
    __syncthreads();
    if constexpr (NEXT) {
      lfrag(0, cur ^ 1, 0);
      mfmas(1);
      sched_substep<0, 0>();
    } else {
      mfmas(1);
    }
  };

  const int nk = (K + BK - 1) / BK;
  using T_ = std::true_type;
  using F_ = std::false_type;
  gload(0);
  lstore(0);
  if (nk > 1) gload(BK);
  __syncthreads();
  lfrag(0, 0, 0);
  int kt = 0;
  for (; kt + 2 < nk; ++kt) kstep(kt, T_{}, T_{});
  if (kt + 1 < nk) kstep(kt++, T_{}, F_{});
  kstep(kt, F_{}, F_{});
  __syncthreads();

  // ---- epilogue: registers -> LDS tile [BM][BNO + 8] (bf16) -> coalesced 16-byte stores
  constexpr int CS = BNO + 8;
  bf16_t* ct = smem;
  // accumulator layout of the 32x32 MFMA: register r of lane l holds
  // row 8*(r/4) + 4*(l/32) + r%4, column l%32 of its 32x32 block
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int jj = 0; jj < (EPI == 0 ? 2 : 4); ++jj) {
      const int col = (EPI == 0 ? wn * 64 + jj * 32 : wn * 128 + jj * 32) + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 128 + i * 32 + (r >> 2) * 8 + lk * 4 + (r & 3);
        float v;
        if (EPI == 0)
          v = silu(acc[i][jj][r]) * acc[i][jj + 2][r];
        else
          v = acc[i][jj][r];
        ct[row * CS + col] = f32_to_bf16(v);
      }
    }
  }
  __syncthreads();
  constexpr int CPR = BNO / 8;  // 16-byte chunks per tile row
  for (int c = tid; c < BM * CPR; c += 256) {
    const int r = c / CPR, cc = (c % CPR) * 8;
    if (r < rows_here && n0 + cc < N)
      *reinterpret_cast<uint4*>(C + static_cast<int64_t>(row_begin + r) * N + n0 + cc) =
          *reinterpret_cast<const uint4*>(ct + r * CS + cc);
  }
}

template <int EPI, bool KTAIL>
hipError_t launch_gemm_t(const bf16_t* A, const int32_t* offsets, const int32_t* tile_off, int groups,
                         int64_t max_tiles, const bf16_t* B0, const bf16_t* B1, int64_t group_stride,
                         int N, int K, bf16_t* C, hipStream_t st) {
  constexpr int BNO = EPI == 0 ? BN / 2 : BN;
  const int64_t nb = cdiv(N, BNO);
  const int64_t grid = cdiv(max_tiles * nb, NXCD) * NXCD;
  // two K stages (128 KiB) or the epilogue's output tile, whichever is larger
  constexpr size_t kMain = 2 * kStageElems * sizeof(bf16_t);
  constexpr size_t kEpi = static_cast<size_t>(BM) * (BNO + 8) * sizeof(bf16_t);
  const size_t lds = kMain > kEpi ? kMain : kEpi;
  static std::atomic<bool> attr_set{false};
  if (!attr_set.load(std::memory_order_acquire)) {
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&grouped_gemm_kernel<EPI, KTAIL>),
        hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    attr_set.store(true, std::memory_order_release);
  }
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((grouped_gemm_kernel<EPI, KTAIL>), dim3(static_cast<unsigned>(grid)), dim3(256), lds,
                     st, A, offsets, tile_off, groups, B0, B1, group_stride, N, K, C);
  return hipGetLastError();
}

template <int EPI>
hipError_t launch_gemm(const bf16_t* A, const int32_t* offsets, const int32_t* tile_off, int groups,
                       int64_t max_tiles, const bf16_t* B0, const bf16_t* B1, int64_t group_stride,
                       int N, int K, bf16_t* C, hipStream_t st) {
  if (K % BK == 0)
    return launch_gemm_t<EPI, false>(A, offsets, tile_off, groups, max_tiles, B0, B1, group_stride,
                                     N, K, C, st);
  return launch_gemm_t<EPI, true>(A, offsets, tile_off, groups, max_tiles, B0, B1, group_stride, N,
                                  K, C, st);
}

}  // namespace

hipError_t launch_gemm_up_bf16(int groups, int d, int Mg, const void* rows,
                               const int32_t* offsets, const int32_t* tile_off, int64_t max_tiles,
                               const void* W_gate, const void* W_up, void* h, hipStream_t st) {
  return launch_gemm<0>(static_cast<const bf16_t*>(rows), offsets, tile_off, groups, max_tiles,
                        static_cast<const bf16_t*>(W_gate), static_cast<const bf16_t*>(W_up),
                        static_cast<int64_t>(Mg) * d, Mg, d, static_cast<bf16_t*>(h), st);
}

hipError_t launch_gemm_down_bf16(int groups, int d, int Mg, const int32_t* offsets,
                                 const int32_t* tile_off, int64_t max_tiles, const void* W_down,
                                 const void* h, void* out, hipStream_t st) {
  return launch_gemm<1>(static_cast<const bf16_t*>(h), offsets, tile_off, groups, max_tiles,
                        static_cast<const bf16_t*>(W_down), nullptr,
                        static_cast<int64_t>(Mg) * d, d, Mg, static_cast<bf16_t*>(out), st);
}

}  // namespace moe

// Grouped expert GEMMs on bf16 MFMA for gfx950 (the SwiGLU experts of "深入理解 MoE (混合专家模型)：
// 稀疏激活与高效扩展" §10.2: h = SiLU(X W_1^T) ⊙ (X W_3^T), out = h W_2^T).
//
// Both products are "TN": every operand row is contiguous along the reduction dimension K, so A
// rows and B rows are read with 16-byte vector loads. A block of 512 threads (8 waves) computes an
// MR x 256 tile with v_mfma_f32_32x32x16_bf16. K advances 64 at a time through two LDS stages (A
// and B slices with XOR-swizzled 16-byte chunks, so fragment reads and stores are bank-conflict-
// free); the next slice is prefetched into registers while the MFMAs run, fragments of the next
// sub-step are read during the current one, and scheduling groups pin the MFMA / LDS / global-load
// interleave.
//
// Gate/up fusion: the B tile's first 128 rows come from W_gate and the last 128 from W_up at the
// same output columns, so a lane holds gate and up values of the same (row, column) and applies
// SiLU(g) * u in registers; h leaves as bf16. The down projection uses 256 plain columns.
//
// Row gather: with a gather list the A rows are read in place from the token matrix (row r of
// the group layout is x[gather[r]]), so the dispatch never materialises the permuted copy of x.
//
// Outputs are written with non-temporal stores: no product re-reads its output soon enough for L2
// to keep it, and streaming them past L2 leaves it to the operand rows that other tiles re-read.
//
// Ragged groups (experts): a group's rows are cut into 256-row tiles; a remainder of 65..128 rows
// becomes a 128-row tile and one of 1..64 rows a 64-row tile, each with its own wave layout, so
// padding rows cost at most half of their tile. The three tile tables (exclusive prefixes per
// group) live on the device; one launch serves all classes: blocks first cover the 256-row tiles
// (consecutive tiles kept on one XCD: blocks are dealt to the 8 XCDs round-robin), then the
// smaller tiles, which the dispatcher starts last so that they fill the final partial round.
#include "moe_internal.h"

#include <math.h>

#include <atomic>
#include <type_traits>

namespace moe {
namespace {

constexpr int BN = 256;  // B rows per tile
constexpr int BK = 64;
constexpr int NXCD = 8;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // native 16-byte value (no struct copy)
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Threads per block of the grouped GEMM: 8 waves, two per SIMD, so one wave's MFMAs cover the
// other's load, store and barrier waits (4 waves also build: -DMOE_GEMM_THREADS=256).
#ifndef MOE_GEMM_THREADS
#define MOE_GEMM_THREADS 512
#endif
constexpr int NT = MOE_GEMM_THREADS;

// Geometry of a tile class with MR rows: waves laid out WM x WN, each owning a block of
// MI x NJ MFMA tiles of 32 x 32.
template <int MR>
struct Geo {
  static constexpr int NW = NT / 64;                              // waves per block
  static constexpr int WM = (NW == 4) ? (MR == 256 ? 2 : 1) : 2;  // waves along rows
  static constexpr int WN = NW / WM;                              // waves along B rows
  static constexpr int WROWS = MR / WM;
  static constexpr int WCOLS = BN / WN;  // B rows per wave
  static constexpr int MI = WROWS / 32;
  static constexpr int NJ = WCOLS / 32;
  static constexpr int RSTEP = NT / 8;      // rows covered by one load pass of the block
  static constexpr int ACH = MR / RSTEP;    // A chunks per thread per k-slice
  static constexpr int BCH = BN / RSTEP;    // B chunks per thread per k-slice
  static constexpr int STAGE = (MR + BN) * BK * 2;  // bytes per LDS stage
  static_assert(MI >= 1 && NJ >= 2 && NJ % 2 == 0 && ACH >= 1, "tile geometry");
};

// element offset of 16-byte chunk `c` (0..7) of row `r` in a [rows][64] swizzled slice
__device__ __forceinline__ int swz(int r, int c) { return r * BK + ((c ^ ((r >> 1) & 7)) << 3); }

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// Instruction-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSgMfma = 0x008, kSgVmemRead = 0x020, kSgDsRead = 0x100, kSgDsWrite = 0x200;

// Schedule of one sub-step: each of the NMF MFMAs is followed by its share of the NR fragment
// reads and of the NX extra instructions of group XMASK (LDS stores or global loads).
template <int NMF, int NR, int XMASK, int NX>
__device__ __forceinline__ void sched_substep() {
  constexpr int RPER = (NR + NMF - 1) / NMF;
  constexpr int XPER = NX > 0 ? (NX + NMF - 1) / NMF : 0;
#pragma unroll
  for (int q = 0; q < NMF; ++q) {
    __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
    if (q * RPER < NR) __builtin_amdgcn_sched_group_barrier(kSgDsRead, RPER, 0);
    if (XPER > 0) __builtin_amdgcn_sched_group_barrier(XMASK, XPER, 0);
  }
  // nothing crosses sub-step boundaries: a sub-step's MFMAs only use fragments read earlier, so
  // the scheduler cannot pull an MFMA next to the LDS read that feeds it
  __builtin_amdgcn_sched_barrier(0);
}

// Schedule of a sub-step with both LDS stores and global loads spread over its MFMAs.
template <int NMF, int NR, int NW, int NL>
__device__ __forceinline__ void sched_substep_wl() {
  constexpr int RPER = (NR + NMF - 1) / NMF;
  constexpr int WPER = (NW + NMF - 1) / NMF;
  constexpr int LPER = (NL + NMF - 1) / NMF;
#pragma unroll
  for (int q = 0; q < NMF; ++q) {
    __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
    if (q * RPER < NR) __builtin_amdgcn_sched_group_barrier(kSgDsRead, RPER, 0);
    if (q * WPER < NW) __builtin_amdgcn_sched_group_barrier(kSgDsWrite, WPER, 0);
    if (q * LPER < NL) __builtin_amdgcn_sched_group_barrier(kSgVmemRead, LPER, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// One MR x 256 output tile of group g: rows [row_begin, row_begin + rows_here), output columns
// [n0, n0 + BNO). EPI 0: SwiGLU (B0 = W_gate, B1 = W_up); EPI 1: plain (B0 = W_down); EPI 2:
// plain with fp32 output (C is then float), stored straight from the accumulators; EPI 3: the
// gate and up pre-activations of EPI 0 stored as fp32 to C and C2; EPI 4: EPI 0 (h to C) after
// storing those pre-activations to C2 and C3.
// KTAIL: K is not a multiple of 64 (the last k-slice is zero-padded). Row r of A starts at
// A + r lda (gathered: A + gather[r] lda), row n of group g's B at B + g group_stride + n ldb, and
// output row r at C + r ldc.
template <int EPI, bool KTAIL, bool GATHER, int MR, bool BKN = false>
__device__ __forceinline__ void run_tile(unsigned char* lds, const bf16_t* __restrict__ A,
                                         int lda, const int32_t* __restrict__ gather,
                                         const bf16_t* __restrict__ B0,
                                         const bf16_t* __restrict__ B1, int64_t group_stride,
                                         int ldb, int N, int K, bf16_t* __restrict__ C, int ldc,
                                         float* __restrict__ C2, float* __restrict__ C3, int g,
                                         int row_begin,
                                         int rows_here, int n0) {
  using G = Geo<MR>;
  constexpr bool PAIRED = EPI == 0 || EPI == 3 || EPI == 4;  // B rows: 128 gate + 128 up
  constexpr bool SWIGLU = EPI == 0 || EPI == 4;               // h = SiLU(gate) * up, bf16
  constexpr int BNO = PAIRED ? BN / 2 : BN;      // output columns per tile
  constexpr int MI = G::MI, NJ = G::NJ, ACH = G::ACH, BCH = G::BCH, RS = G::RSTEP;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / G::WN, wn = wave % G::WN;

  // ---- global loads: thread `tid` moves chunk (tid & 7) of rows r0 + RS i of the A slice
  // (i < ACH) and of the B slice (i < BCH). Addresses are uniform tile bases plus 32-bit byte
  // offsets fixed over K (gathered A rows: one 64-bit row address each); rows past the group (A)
  // or past N (B) re-read the last valid row and never reach a stored output.
  const int r0 = tid >> 3, kc_t = (tid & 7) * 8;
  const char* a_base = reinterpret_cast<const char*>(A + static_cast<int64_t>(row_begin) * lda);
  const char* a_row[GATHER ? ACH : 1];
  if constexpr (GATHER) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int t = gather[row_begin + min(i * RS + r0, rows_here - 1)];
      a_row[i] = reinterpret_cast<const char*>(A + static_cast<int64_t>(t) * lda + kc_t);
    }
  }
  const bf16_t* Bg0 = B0 + static_cast<int64_t>(g) * group_stride + static_cast<int64_t>(n0) * ldb;
  const bf16_t* Bg1 =
      PAIRED ? B1 + static_cast<int64_t>(g) * group_stride + static_cast<int64_t>(n0) * ldb : Bg0;
  const char* b_base0 = reinterpret_cast<const char*>(Bg0);
  const char* b_base1 = reinterpret_cast<const char*>(Bg1);
  const int b_rows = min(PAIRED ? BN / 2 : BN, N - n0);
  uint32_t a_off[ACH], b_off[BCH];
#pragma unroll
  for (int i = 0; i < ACH; ++i)
    a_off[i] = static_cast<uint32_t>((min(i * RS + r0, rows_here - 1) * lda + kc_t) * 2);
#pragma unroll
  for (int i = 0; i < BCH; ++i) {
    const int r = i * RS + r0;
    const int rb_ = PAIRED ? (r & (BN / 2 - 1)) : r;
    b_off[i] = static_cast<uint32_t>((min(rb_, b_rows - 1) * ldb + kc_t) * 2);
  }
  // BKN: B is [K][N] (N contiguous, row stride ldb; with B1, rows K/2.. come from B1): chunk
  // i * NT + tid of a 64 x 256 slice is row 16 i + tid / 32, columns n0 + 8 (tid % 32). Nothing
  // loaded is zeroed: a column past N only reaches output columns that are never stored, and a
  // row past K (clamped to row K - 1, so finite) only meets A chunks that are zero.
  static_assert(!BKN || (EPI == 2 && NT == 512), "K-major B is wired for the fp32-output products");
  const char* bk0 = reinterpret_cast<const char*>(B0 + static_cast<int64_t>(g) * group_stride);
  const int khalf = B1 != nullptr ? K / 2 : K;
  const uint32_t ldb2 = static_cast<uint32_t>(ldb) * 2u;
  // byte distance from row kk of B0's group to row kk - K/2 of B1's (rows K/2.. only)
  const int64_t dB = (BKN && B1 != nullptr)
                         ? (reinterpret_cast<const char*>(B1 + static_cast<int64_t>(g) * group_stride) -
                            bk0) - static_cast<int64_t>(khalf) * ldb2
                         : 0;
  const int bk_r = tid >> 5;
  const uint32_t bk_cb = static_cast<uint32_t>(min(n0 + (tid & 31) * 8, N - 8)) * 2u;
  u32x4 ra[ACH], rb[BCH];
  auto gload = [&](int k0) __attribute__((always_inline)) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
    const bool in = !KTAIL || k0 + kc_t < K;
    // a chunk past K re-reads the row's last chunk and is then zeroed
    const uint32_t kb = static_cast<uint32_t>((in ? k0 : K - 8 - kc_t) * 2);
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const char* ap = GATHER ? a_row[GATHER ? i : 0] + kb : a_base + (a_off[i] + kb);
      const u32x4 v = *reinterpret_cast<const u32x4*>(ap);
      ra[i] = KTAIL ? (in ? v : zero) : v;
    }
    if constexpr (BKN) {
#pragma unroll
      for (int i = 0; i < BCH; ++i) {
        const int kk = KTAIL ? min(k0 + 16 * i + bk_r, K - 1) : k0 + 16 * i + bk_r;
        const char* bp = bk0 + (static_cast<uint32_t>(kk) * ldb2 + bk_cb) + (kk >= khalf ? dB : 0);
        rb[i] = *reinterpret_cast<const u32x4*>(bp);
      }
    } else {
#pragma unroll
      for (int i = 0; i < BCH; ++i) {
        const char* bb = (PAIRED && i >= BCH / 2) ? b_base1 : b_base0;
        const u32x4 v = *reinterpret_cast<const u32x4*>(bb + (b_off[i] + kb));
        rb[i] = KTAIL ? (in ? v : zero) : v;
      }
    }
  };
  // LDS byte offset of this thread's chunk of row r0; row r0 + RS i sits RS * 128 B further on
  // (the swizzle term depends on (r >> 1) & 7, which is the same for all i)
  const uint32_t st_off = static_cast<uint32_t>(swz(r0, tid & 7) * 2);
  constexpr uint32_t kStageBytes = G::STAGE, kBBytes = MR * BK * 2;
  auto lstore = [&](int stage) __attribute__((always_inline)) {
    unsigned char* sa = lds + stage * kStageBytes + st_off;
#pragma unroll
    for (int i = 0; i < ACH; ++i) *reinterpret_cast<u32x4*>(sa + i * RS * BK * 2) = ra[i];
    if constexpr (BKN) {
      // [64 k][256 n] slice, 512-byte rows, 16-byte chunk c of row r at chunk c ^ 4 (r & 3)
      // (a 64-byte step, so the 32-byte pieces of a transposing read's two column halves land on
      // distinct banks); a thread's chunks are rows 16 apart, so r & 3 is the same for all of them
      unsigned char* sb = lds + stage * kStageBytes + kBBytes + bk_r * 512 +
                          (((tid & 31) ^ ((bk_r & 3) << 2)) << 4);
#pragma unroll
      for (int i = 0; i < BCH; ++i) *reinterpret_cast<u32x4*>(sb + i * 16 * 512) = rb[i];
    } else {
#pragma unroll
      for (int i = 0; i < BCH; ++i)
        *reinterpret_cast<u32x4*>(sa + kBBytes + i * RS * BK * 2) = rb[i];
    }
  };

  f32x16 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // ---- MFMA fragments: lane l reads row (l % 32) of a 32-row block, k-chunk 2*sub + l/32.
  // Every block starts at a multiple of 32 rows, so the swizzle term is the lane's own.
  const int l32 = lane & 31, lk = lane >> 5, sw = (l32 >> 1) & 7;
  uint32_t fo[4];
#pragma unroll
  for (int sub = 0; sub < 4; ++sub)
    fo[sub] = static_cast<uint32_t>((l32 * BK + (((sub * 2 + lk) ^ sw) << 3)) * 2);
  // B-tile rows of this wave's 32-column blocks: for SwiGLU the first half are gate rows, the
  // second half the up rows of the same output columns
  int brow[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j)
    brow[j] = PAIRED ? ((j < NJ / 2 ? 0 : BN / 2) + wn * (G::WCOLS / 2) + (j % (NJ / 2)) * 32)
                       : (wn * G::WCOLS + j * 32);
  // BKN fragments by transposing reads (ds_read_b64_tr_b16): in each group of 16 lanes, lane
  // 4 q + a reads 4 columns (n_base + 4 a ..) of row k_base + q, and lane i receives the 4 rows
  // k_base .. k_base + 3 of column n_base + i. Lane l's 32x32x16 B operand (8 k of column
  // l % 32) is two such reads, rows 16 sub + 8 (l / 32) + {0..3} and {4..7}.
  uint32_t tb_off[BKN ? NJ : 1];
  if constexpr (BKN) {
    const int g4 = lane >> 4, i16 = lane & 15;
    const int trow = 8 * (g4 >> 1) + (i16 >> 2);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int col = brow[j] + 16 * (g4 & 1) + 4 * (i16 & 3);
      tb_off[j] = static_cast<uint32_t>(kBBytes + trow * 512 +
                                        (((col >> 3) ^ ((i16 >> 2) << 2)) << 4) +
                                        (((col >> 2) & 1) << 3));
    }
  }
  bf16x8 fa[2][MI], fb[2][NJ];
  auto lfrag = [&](int set, int stage, int sub) __attribute__((always_inline)) {
    const unsigned char* sa = lds + stage * kStageBytes + fo[sub];
#pragma unroll
    for (int i = 0; i < MI; ++i)
      fa[set][i] = *reinterpret_cast<const bf16x8*>(sa + (wm * G::WROWS + i * 32) * BK * 2);
    if constexpr (BKN) {
      typedef short v4i16 __attribute__((ext_vector_type(4)));
      typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const unsigned char* pb = lds + stage * kStageBytes + tb_off[j] + sub * 16 * 512;
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(pb));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(pb + 4 * 512));
        fb[set][j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    } else {
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        fb[set][j] = *reinterpret_cast<const bf16x8*>(sa + kBBytes + brow[j] * BK * 2);
    }
  };
  auto mfmas = [&](int set) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[set][i], fb[set][j], acc[i][j], 0, 0, 0);
  };
  constexpr int NMF = MI * NJ, NR = MI + (BKN ? 2 * NJ : NJ), NX = ACH + BCH;

  // ---- one k-step (64 of K) = 4 sub-steps on stage `cur`:
  //   sub 0: read fragments of sub 1, store stage cur^1 (no wave reads it since the last
  //          barrier), then load k-step +2 into the freed registers | MFMAs of sub 0
  //   sub 1: read fragments of sub 2                                | MFMAs of sub 1
  //   sub 2: read fragments of sub 3                                | MFMAs of sub 2
  //   barrier (stage cur^1 complete; every read of stage cur issued)
  //   sub 3: read fragments of sub 0 of stage cur^1                 | MFMAs of sub 3
  // A global load has four sub-steps to land before its LDS store; no LDS read waits on a
  // barrier.
  auto kstep = [&](int kt, auto has_next, auto has_load) __attribute__((always_inline)) {
    constexpr bool NEXT = decltype(has_next)::value;  // a following k-step exists
    constexpr bool LOAD = decltype(has_load)::value;  // k-step kt + 2 exists
    const int cur = kt & 1;
    lfrag(1, cur, 1);
    mfmas(0);
    if constexpr (NEXT && LOAD) {
      lstore(cur ^ 1);
      gload((kt + 2) * BK);
      sched_substep_wl<NMF, NR, NX, NX>();
    } else if constexpr (NEXT) {
      lstore(cur ^ 1);
      sched_substep<NMF, NR, kSgDsWrite, NX>();
    } else {
      sched_substep<NMF, NR, 0, 0>();
    }
    lfrag(0, cur, 2);
    mfmas(1);
    sched_substep<NMF, NR, 0, 0>();
    lfrag(1, cur, 3);
    mfmas(0);
    sched_substep<NMF, NR, 0, 0>();
    __syncthreads();
    if constexpr (NEXT) {
      lfrag(0, cur ^ 1, 0);
      mfmas(1);
      sched_substep<NMF, NR, 0, 0>();
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
  if constexpr (EPI == 2) {
    // fp32 output: each lane stores its accumulators (32 consecutive columns per row and wave)
    float* C32 = reinterpret_cast<float*>(C);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int col = n0 + wn * G::WCOLS + j * 32 + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wm * G::WROWS + i * 32 + (r >> 2) * 8 + lk * 4 + (r & 3);
          if (row < rows_here && col < N)
            __builtin_nontemporal_store(acc[i][j][r], &C32[static_cast<int64_t>(row_begin + row) * ldc + col]);
        }
      }
    return;
  }
  if constexpr (EPI == 3 || EPI == 4) {
    // fp32 gate and up pre-activations of the same output columns: to C and C2 (EPI 3), or to C2
    // and C3 ahead of the SwiGLU epilogue that writes h to C (EPI 4)
    float* Cg = EPI == 3 ? reinterpret_cast<float*>(C) : C2;
    float* Cu = EPI == 3 ? C2 : C3;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int jj = 0; jj < NJ / 2; ++jj) {
        const int col = n0 + wn * (G::WCOLS / 2) + jj * 32 + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wm * G::WROWS + i * 32 + (r >> 2) * 8 + lk * 4 + (r & 3);
          if (row < rows_here && col < N) {
            const int64_t o = static_cast<int64_t>(row_begin + row) * ldc + col;
            __builtin_nontemporal_store(acc[i][jj][r], &Cg[o]);
            __builtin_nontemporal_store(acc[i][jj + NJ / 2][r], &Cu[o]);
          }
        }
      }
    if constexpr (EPI == 3) return;
  }
  __syncthreads();

  // ---- epilogue: registers -> LDS tile [MR][BNO + 8] (bf16) -> coalesced 16-byte stores
  constexpr int CS = BNO + 8;
  bf16_t* ct = reinterpret_cast<bf16_t*>(lds);
  // accumulator layout of the 32x32 MFMA: register r of lane l holds
  // row 8*(r/4) + 4*(l/32) + r%4, column l%32 of its 32x32 block
#pragma unroll
  for (int i = 0; i < MI; ++i) {
#pragma unroll
    for (int jj = 0; jj < (SWIGLU ? NJ / 2 : NJ); ++jj) {
      const int col = (SWIGLU ? wn * (G::WCOLS / 2) : wn * G::WCOLS) + jj * 32 + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * G::WROWS + i * 32 + (r >> 2) * 8 + lk * 4 + (r & 3);
        float v;
        if (SWIGLU)
          v = silu(acc[i][jj][r]) * acc[i][jj + NJ / 2][r];
        else
          v = acc[i][jj][r];
        ct[row * CS + col] = f32_to_bf16(v);
      }
    }
  }
  __syncthreads();
  constexpr int CPR = BNO / 8;  // 16-byte chunks per tile row
  for (int c = tid; c < MR * CPR; c += NT) {
    const int r = c / CPR, cc = (c % CPR) * 8;
    if (r < rows_here && n0 + cc < N)
      __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(ct + r * CS + cc),
                                  reinterpret_cast<u32x4*>(C + static_cast<int64_t>(row_begin + r) * ldc + n0 + cc));
  }
}

// Largest g with table[g] * nb_count <= L (table is non-decreasing, table[0] = 0).
__device__ __forceinline__ int find_group(const int32_t* __restrict__ table, int groups,
                                          int nb_count, int64_t L) {
  int lo = 0, hi = groups;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (static_cast<int64_t>(table[mid]) * nb_count <= L) lo = mid; else hi = mid;
  }
  return lo;
}

// tile_off: three tables of groups + 1 entries: 256-row tiles, 128-row tiles, 64-row tiles.
// Blocks [0, main_blocks) serve the 256-row tiles, the rest the smaller ones.
template <int EPI, bool KTAIL, bool GATHER, bool BKN = false>
__global__ __launch_bounds__(NT, 1) void grouped_gemm_kernel(
    const bf16_t* __restrict__ A, const int32_t* __restrict__ gather,
    const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ tile_off, int groups, int main_blocks,
    const bf16_t* __restrict__ B0, const bf16_t* __restrict__ B1, int64_t group_stride, int N,
    int K, bf16_t* __restrict__ C, float* __restrict__ C2, float* __restrict__ C3) {
  constexpr int BNO = (EPI == 0 || EPI == 3 || EPI == 4) ? BN / 2 : BN;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int nb_count = (N + BNO - 1) / BNO;
  const int32_t* t256 = tile_off;
  const int32_t* t128 = tile_off + (groups + 1);
  const int32_t* t64 = tile_off + 2 * (groups + 1);
  if (static_cast<int>(blockIdx.x) < main_blocks) {
    const int64_t ntiles = static_cast<int64_t>(t256[groups]) * nb_count;
    const int64_t q = (ntiles + NXCD - 1) / NXCD;
    const int64_t L = static_cast<int64_t>(blockIdx.x % NXCD) * q + blockIdx.x / NXCD;
    if (blockIdx.x / NXCD >= q || L >= ntiles) return;
    const int g = find_group(t256, groups, nb_count, L);
    const int mt_g = t256[g + 1] - t256[g];
    const int64_t local = L - static_cast<int64_t>(t256[g]) * nb_count;
    const int nb = static_cast<int>(local / mt_g), mt = static_cast<int>(local % mt_g);
    const int row_begin = offsets[g] + mt * 256;
    const int rows = min(256, offsets[g + 1] - row_begin);
    run_tile<EPI, KTAIL, GATHER, 256, BKN>(lds, A, K, gather, B0, B1, group_stride, BKN ? N : K, N,
                                           K, C, N, C2,
                                      C3, g, row_begin, rows, nb * BNO);
    return;
  }
  // a group's remainder tile (at most one per group and class): n-blocks in order
  int64_t L = static_cast<int64_t>(blockIdx.x) - main_blocks;
  const int64_t n128 = static_cast<int64_t>(t128[groups]) * nb_count;
  const int64_t n64 = static_cast<int64_t>(t64[groups]) * nb_count;
  const int32_t* table = L < n128 ? t128 : t64;
  if (L >= n128) {
    L -= n128;
    if (L >= n64) return;
  }
  const int g = find_group(table, groups, nb_count, L);
  const int64_t local = L - static_cast<int64_t>(table[g]) * nb_count;
  const int rows_g = offsets[g + 1] - offsets[g];
  const int row_begin = offsets[g] + (rows_g & ~255);
  const int rows = rows_g & 255;
  const int n0 = static_cast<int>(local) * BNO;
  if (table == t128)
    run_tile<EPI, KTAIL, GATHER, 128, BKN>(lds, A, K, gather, B0, B1, group_stride, BKN ? N : K, N,
                                           K, C, N, C2,
                                      C3, g, row_begin, rows, n0);
  else
    run_tile<EPI, KTAIL, GATHER, 64, BKN>(lds, A, K, gather, B0, B1, group_stride, BKN ? N : K, N,
                                          K, C, N, C2,
                                     C3, g, row_begin, rows, n0);
}

// Weight gradients: C_g [Ma][Nb] (fp32) = sum over k in [64 kt[g], 64 kt[g+1]) of A[m][k] B[n][k],
// for the operands A [Ma][lda] and B [Nb][ldb] whose columns are the rows of the groups, each
// group padded with zeros to a multiple of 64 (so no k-slice is partial). 256 x 256 output tiles
// in bands of 8 m-tiles (neighbouring tiles share A and B slabs), dealt to the XCDs in runs; a group
// without rows gets zeros.
__global__ __launch_bounds__(NT, 1) void wgrad_gemm_kernel(const bf16_t* __restrict__ A, int lda,
                                                           const bf16_t* __restrict__ B, int ldb,
                                                           const int32_t* __restrict__ kt,
                                                           int groups, int Ma, int Nb,
                                                           float* __restrict__ C) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int mt = (Ma + 255) / 256, nt = (Nb + 255) / 256;
  const int64_t per_group = static_cast<int64_t>(mt) * nt;
  const int64_t ntiles = static_cast<int64_t>(groups) * per_group;
  const int64_t q = (ntiles + NXCD - 1) / NXCD;
  const int64_t L = static_cast<int64_t>(blockIdx.x % NXCD) * q + blockIdx.x / NXCD;
  if (blockIdx.x / NXCD >= q || L >= ntiles) return;
  const int g = static_cast<int>(L / per_group);
  const int local = static_cast<int>(L % per_group);
  // bands of kWgBand m-tiles, n fastest within a band's column: the 32 tiles an XCD runs at
  // once span 8 m x 4 n and read 12 operand slabs instead of 33 (a narrower last band)
  constexpr int kWgBand = 8;
  const int band = local / (kWgBand * nt), w = local % (kWgBand * nt);
  const int bw = min(kWgBand, mt - band * kWgBand);
  const int m0 = (band * kWgBand + w % bw) * 256, n0 = (w / bw) * 256;
  const int k0 = 64 * kt[g], K = 64 * (kt[g + 1] - kt[g]);
  float* Cg = C + static_cast<int64_t>(g) * Ma * Nb;
  if (K == 0) {
    for (int c = threadIdx.x; c < 256 * 64; c += NT) {
      const int r = m0 + c / 64, cc = n0 + (c % 64) * 4;
      if (r < Ma && cc < Nb)
        *reinterpret_cast<float4*>(Cg + static_cast<int64_t>(r) * Nb + cc) =
            make_float4(0.f, 0.f, 0.f, 0.f);
    }
    return;
  }
  run_tile<2, false, false, 256>(lds, A + k0, lda, nullptr, B + k0, nullptr, 0, ldb, Nb, K,
                                 reinterpret_cast<bf16_t*>(Cg), Nb, nullptr, nullptr, 0, m0,
                                 min(256, Ma - m0), n0);
}

template <int EPI, bool KTAIL, bool GATHER, bool BKN = false>
hipError_t launch_gemm_t(const bf16_t* A, const int32_t* gather, const int32_t* offsets,
                         const int32_t* tile_off,
                         int groups, int64_t max_tiles, const bf16_t* B0, const bf16_t* B1,
                         int64_t group_stride, int N, int K, bf16_t* C, float* C2,
                         float* C3, hipStream_t st) {
  constexpr int BNO = (EPI == 0 || EPI == 3 || EPI == 4) ? BN / 2 : BN;
  const int64_t nb = cdiv(N, BNO);
  // the 256-row tiles, then at most one 128-row and one 64-row tile per group
  const int64_t main_blocks = cdiv(max_tiles * nb, NXCD) * NXCD;
  const int64_t grid = main_blocks + 2 * static_cast<int64_t>(groups) * nb;
  // two K stages of the 256-row class or its epilogue tile, whichever is larger
  constexpr size_t kMain = 2 * Geo<256>::STAGE;
  constexpr size_t kEpi = static_cast<size_t>(256) * (BNO + 8) * sizeof(bf16_t);
  const size_t lds = kMain > kEpi ? kMain : kEpi;
  static std::atomic<bool> attr_set{false};
  if (!attr_set.load(std::memory_order_acquire)) {
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&grouped_gemm_kernel<EPI, KTAIL, GATHER, BKN>),
        hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    attr_set.store(true, std::memory_order_release);
  }
  if (max_tiles <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((grouped_gemm_kernel<EPI, KTAIL, GATHER, BKN>), dim3(static_cast<unsigned>(grid)),
                     dim3(NT), lds, st, A, gather, offsets, tile_off, groups,
                     static_cast<int>(main_blocks), B0, B1, group_stride, N, K, C, C2, C3);
  return hipGetLastError();
}

template <int EPI, bool GATHER, bool BKN = false>
hipError_t launch_gemm(const bf16_t* A, const int32_t* gather, const int32_t* offsets,
                       const int32_t* tile_off, int groups, int64_t max_tiles, const bf16_t* B0,
                       const bf16_t* B1, int64_t group_stride, int N, int K, bf16_t* C,
                       hipStream_t st, float* C2 = nullptr, float* C3 = nullptr) {
  if (K % BK == 0)
    return launch_gemm_t<EPI, false, GATHER, BKN>(A, gather, offsets, tile_off, groups, max_tiles,
                                                  B0, B1, group_stride, N, K, C, C2, C3, st);
  return launch_gemm_t<EPI, true, GATHER, BKN>(A, gather, offsets, tile_off, groups, max_tiles, B0,
                                               B1, group_stride, N, K, C, C2, C3, st);
}

}  // namespace

hipError_t launch_gemm_up_bf16(int groups, int d, int Mg, const void* rows,
                               const int32_t* gather, const int32_t* offsets,
                               const int32_t* tile_off, int64_t max_tiles, const void* W_gate,
                               const void* W_up, void* h, hipStream_t st) {
  const bf16_t* A = static_cast<const bf16_t*>(rows);
  const bf16_t* Wg = static_cast<const bf16_t*>(W_gate);
  const bf16_t* Wu = static_cast<const bf16_t*>(W_up);
  const int64_t gs = static_cast<int64_t>(Mg) * d;
  bf16_t* H = static_cast<bf16_t*>(h);
  if (gather != nullptr)
    return launch_gemm<0, true>(A, gather, offsets, tile_off, groups, max_tiles, Wg, Wu, gs, Mg, d,
                                H, st);
  return launch_gemm<0, false>(A, nullptr, offsets, tile_off, groups, max_tiles, Wg, Wu, gs, Mg, d,
                               H, st);
}

// G[r] = A_r W_gate[g]^T and U[r] = A_r W_up[g]^T in fp32 (A_r = rows[gather[r]] when gather !=
// NULL): the gate/up tile of the SwiGLU GEMM with the pre-activations stored instead of h (the
// backward's recompute)
hipError_t launch_gemm_gu_f32out_bf16(int groups, int d, int Mg, const void* rows,
                                      const int32_t* gather, const int32_t* offsets,
                                      const int32_t* tile_off, int64_t max_tiles,
                                      const void* W_gate, const void* W_up, float* G, float* U,
                                      hipStream_t st) {
  const bf16_t* A = static_cast<const bf16_t*>(rows);
  const bf16_t* Wg = static_cast<const bf16_t*>(W_gate);
  const bf16_t* Wu = static_cast<const bf16_t*>(W_up);
  const int64_t gs = static_cast<int64_t>(Mg) * d;
  bf16_t* Gp = reinterpret_cast<bf16_t*>(G);  // holds floats (EPI 3)
  if (gather != nullptr)
    return launch_gemm<3, true>(A, gather, offsets, tile_off, groups, max_tiles, Wg, Wu, gs, Mg, d,
                                Gp, st, U);
  return launch_gemm<3, false>(A, nullptr, offsets, tile_off, groups, max_tiles, Wg, Wu, gs, Mg, d,
                               Gp, st, U);
}

// The SwiGLU GEMM of launch_gemm_up_bf16 that also stores the fp32 gate and up pre-activations
// G[r] and U[r] (the values launch_gemm_gu_f32out_bf16 computes, from the same accumulators), so
// that a backward can take them instead of recomputing them; h is unchanged.
hipError_t launch_gemm_up_save_bf16(int groups, int d, int Mg, const void* rows,
                                    const int32_t* gather, const int32_t* offsets,
                                    const int32_t* tile_off, int64_t max_tiles, const void* W_gate,
                                    const void* W_up, void* h, float* G, float* U,
                                    hipStream_t st) {
  const bf16_t* A = static_cast<const bf16_t*>(rows);
  const bf16_t* Wg = static_cast<const bf16_t*>(W_gate);
  const bf16_t* Wu = static_cast<const bf16_t*>(W_up);
  const int64_t gs = static_cast<int64_t>(Mg) * d;
  bf16_t* H = static_cast<bf16_t*>(h);
  if (gather != nullptr)
    return launch_gemm<4, true>(A, gather, offsets, tile_off, groups, max_tiles, Wg, Wu, gs, Mg, d,
                                H, st, G, U);
  return launch_gemm<4, false>(A, nullptr, offsets, tile_off, groups, max_tiles, Wg, Wu, gs, Mg, d,
                               H, st, G, U);
}

// C[r] = A_r B_g^T for the rows of group g (A_r = rows[gather[r]] when gather != NULL): the plain
// epilogue with any N and K (the backward recomputes the gate and up pre-activations with it)
// (fp32 output)
hipError_t launch_gemm_plain_bf16(int groups, const void* rows, const int32_t* gather,
                                  const int32_t* offsets, const int32_t* tile_off,
                                  int64_t max_tiles, const void* B, int64_t group_stride, int N,
                                  int K, void* C, hipStream_t st) {
  const bf16_t* A = static_cast<const bf16_t*>(rows);
  const bf16_t* Bp = static_cast<const bf16_t*>(B);
  bf16_t* Cp = static_cast<bf16_t*>(C);  // holds floats (EPI 2)
  if (gather != nullptr)
    return launch_gemm<2, true>(A, gather, offsets, tile_off, groups, max_tiles, Bp, nullptr,
                                group_stride, N, K, Cp, st);
  return launch_gemm<2, false>(A, nullptr, offsets, tile_off, groups, max_tiles, Bp, nullptr,
                               group_stride, N, K, Cp, st);
}

// C[r] = A_r B_g for the rows of group g with B_g [K][N] row-major (N contiguous; no transposed
// copy): group g's B is B0 + g group_stride, and with B1 != NULL its rows K/2 .. K - 1 are those
// of B1 + g group_stride (so [dG dU] [W_gate; W_up] runs over K = 2M in one launch). fp32 output.
hipError_t launch_gemm_kn_bf16(int groups, const void* rows, const int32_t* gather,
                               const int32_t* offsets, const int32_t* tile_off, int64_t max_tiles,
                               const void* B0, const void* B1, int64_t group_stride, int N, int K,
                               float* C, hipStream_t st) {
  const bf16_t* A = static_cast<const bf16_t*>(rows);
  const bf16_t* b0 = static_cast<const bf16_t*>(B0);
  const bf16_t* b1 = static_cast<const bf16_t*>(B1);
  bf16_t* Cp = reinterpret_cast<bf16_t*>(C);  // holds floats (EPI 2)
  // 16-byte column chunks, and a group's row offsets (K rows of N) in 32 bits
  if (N < 8 || N % 8 != 0 || static_cast<int64_t>(K) * N * 2 >= (int64_t{1} << 32))
    return hipErrorInvalidValue;
  if (gather != nullptr)
    return launch_gemm<2, true, true>(A, gather, offsets, tile_off, groups, max_tiles, b0, b1,
                                      group_stride, N, K, Cp, st);
  return launch_gemm<2, false, true>(A, nullptr, offsets, tile_off, groups, max_tiles, b0, b1,
                                     group_stride, N, K, Cp, st);
}

// C_g = A_g B_g^T over each group's zero-padded column range (weight gradients, fp32 output)
hipError_t launch_gemm_wgrad_bf16(const void* A, int lda, const void* B, int ldb,
                                  const int32_t* kt, int groups, int Ma, int Nb, float* C,
                                  hipStream_t st) {
  constexpr size_t lds = 2 * Geo<256>::STAGE;
  static std::atomic<bool> attr_set{false};
  if (!attr_set.load(std::memory_order_acquire)) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&wgrad_gemm_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
    attr_set.store(true, std::memory_order_release);
  }
  const int64_t tiles = static_cast<int64_t>(groups) * cdiv(Ma, 256) * cdiv(Nb, 256);
  if (tiles <= 0) return hipSuccess;
  const int64_t grid = cdiv(tiles, NXCD) * NXCD;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(wgrad_gemm_kernel, dim3(static_cast<unsigned>(grid)), dim3(NT), lds, st,
                     static_cast<const bf16_t*>(A), lda, static_cast<const bf16_t*>(B), ldb, kt,
                     groups, Ma, Nb, C);
  return hipGetLastError();
}

hipError_t launch_gemm_down_bf16(int groups, int d, int Mg, const int32_t* offsets,
                                 const int32_t* tile_off, int64_t max_tiles, const void* W_down,
                                 const void* h, void* out, hipStream_t st) {
  return launch_gemm<1, false>(static_cast<const bf16_t*>(h), nullptr, offsets, tile_off, groups,
                               max_tiles, static_cast<const bf16_t*>(W_down), nullptr,
                               static_cast<int64_t>(Mg) * d, d, Mg, static_cast<bf16_t*>(out), st);
}

}  // namespace moe

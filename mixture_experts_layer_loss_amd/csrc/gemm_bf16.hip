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
// The forward products with K of 2..128 k-slices run persistent blocks over the 256-row tiles: the
// k-step pipeline runs on from one tile into the block's next, so a tile costs no launch, lookup
// or first-load round trip (run_tiles_persistent); the remainder tiles below stay one per block.
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

// SiLU(z) = z / (1 + e^-z), with the hardware reciprocal (about 1 ulp) in place of a full division
__device__ __forceinline__ float silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

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
  // The 64- and 128-row tiles keep two k-slices in registers (their k-steps are short, so one
  // k-step is not enough to cover a load from HBM): slot q holds k-slices q, q + 2, ...
  constexpr bool RING = MR < 256;
  u32x4 rga[RING ? 2 : 1][ACH], rgb[RING ? 2 : 1][BCH];
  auto gload_to = [&](int k0, auto slot) __attribute__((always_inline)) {
    constexpr int S = decltype(slot)::value;
    u32x4 (&ra)[ACH] = rga[S];
    u32x4 (&rb)[BCH] = rgb[S];
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
  auto lstore_from = [&](int stage, auto slot) __attribute__((always_inline)) {
    constexpr int S = decltype(slot)::value;
    const u32x4 (&ra)[ACH] = rga[S];
    const u32x4 (&rb)[BCH] = rgb[S];
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
  // MFMA order: the B fragment runs backwards on odd row blocks, so consecutive MFMAs share an
  // operand across the row-block boundary too (fewer operand bits switch: a power-limited clock)
  auto mfmas = [&](int set) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) {
        const int j = (i & 1) ? NJ - 1 - jj : jj;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[set][i], fb[set][j], acc[i][j], 0, 0, 0);
      }
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
  // slot: the register slot holding k-slice kt + 1 (always 0 without the ring); with the ring the
  // k-step loads k-slice kt + 3 into it once it is stored, else k-slice kt + 2
  auto kstep = [&](int kt, auto has_next, auto has_load, auto slot, int nk) __attribute__((always_inline)) {
    constexpr bool NEXT = decltype(has_next)::value;  // a following k-step exists
    constexpr bool LOAD = decltype(has_load)::value;  // the k-slice to load exists
    const int cur = kt & 1;
    lfrag(1, cur, 1);
    mfmas(0);
    if constexpr (NEXT && LOAD) {
      lstore_from(cur ^ 1, slot);
      gload_to((RING ? min(kt + 3, nk - 1) : kt + 2) * BK, slot);
      sched_substep_wl<NMF, NR, NX, NX>();
    } else if constexpr (NEXT) {
      lstore_from(cur ^ 1, slot);
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
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, RING ? 1 : 0>;
  if constexpr (RING) {
    // unconditional (clamped) loads keep the wait for slot 0 from covering slot 1's loads
    gload_to(0, S0{});
    gload_to(min(1, nk - 1) * BK, S1{});
    lstore_from(0, S0{});
    gload_to(min(2, nk - 1) * BK, S0{});
    __syncthreads();
    lfrag(0, 0, 0);
    // k-step kt stores k-slice kt + 1 (slot (kt + 1) % 2) and loads k-slice kt + 3 into that slot;
    // past the last k-slice it loads the last one again (in bounds, never stored)
    int kt = 0;
    for (; kt + 2 < nk; kt += 2) {
      kstep(kt, T_{}, T_{}, S1{}, nk);
      kstep(kt + 1, T_{}, T_{}, S0{}, nk);
    }
    if (kt + 1 < nk) {
      kstep(kt, T_{}, F_{}, S1{}, nk);
      kstep(kt + 1, F_{}, F_{}, S0{}, nk);
    } else {
      kstep(kt, F_{}, F_{}, S1{}, nk);
    }
  } else {
    gload_to(0, S0{});
    lstore_from(0, S0{});
    if (nk > 1) gload_to(BK, S0{});
    __syncthreads();
    lfrag(0, 0, 0);
    int kt = 0;
    for (; kt + 2 < nk; ++kt) kstep(kt, T_{}, T_{}, S0{}, nk);
    if (kt + 1 < nk) kstep(kt++, T_{}, F_{}, S0{}, nk);
    kstep(kt, F_{}, F_{}, S0{}, nk);
  }
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

// Remainder tile L (counted over the 128-row tiles, then the 64-row ones): a group's rows past its
// 256-row tiles, at most one tile per group and class; n-blocks in order.
template <int EPI, bool KTAIL, bool GATHER, bool BKN>
__device__ __forceinline__ void run_remainder_tile(
    unsigned char* lds, int64_t L, const bf16_t* __restrict__ A,
    const int32_t* __restrict__ gather, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ tile_off, int groups, const bf16_t* __restrict__ B0,
    const bf16_t* __restrict__ B1, int64_t group_stride, int N, int K, bf16_t* __restrict__ C,
    float* __restrict__ C2, float* __restrict__ C3) {
  constexpr int BNO = (EPI == 0 || EPI == 3 || EPI == 4) ? BN / 2 : BN;
  const int nb_count = (N + BNO - 1) / BNO;
  const int32_t* t128 = tile_off + (groups + 1);
  const int32_t* t64 = tile_off + 2 * (groups + 1);
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
                                           K, C, N, C2, C3, g, row_begin, rows, n0);
  else
    run_tile<EPI, KTAIL, GATHER, 64, BKN>(lds, A, K, gather, B0, B1, group_stride, BKN ? N : K, N,
                                          K, C, N, C2, C3, g, row_begin, rows, n0);
}

// K chunk ks of `split` of remainder tile L of a plain long-K product (the forward down
// projection, EPI 1, or a backward product with a K-major B, EPI 2): the tile's rows times the
// chunk's k-slices, as fp32 partial sums into part[((ks groups + g) 128 + r) N + n] for remainder
// row r of group g. Every chunk is a whole number of k-slices except perhaps the last (KTAIL);
// with two B matrices (rows K/2.. from B1) the two chunks are the halves, K/2 a multiple of 64.
// finish_split_kernel adds the chunks.
template <int EPI, bool KTAIL, bool GATHER, bool BKN>
__device__ __forceinline__ void run_remainder_split(
    unsigned char* lds, int64_t L, int ks, int split, const bf16_t* __restrict__ A,
    const int32_t* __restrict__ gather, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ tile_off, int groups, const bf16_t* __restrict__ B0,
    const bf16_t* __restrict__ B1, int64_t group_stride, int N, int K, float* __restrict__ part) {
  const int nb_count = (N + BN - 1) / BN;
  const int32_t* t128 = tile_off + (groups + 1);
  const int32_t* t64 = tile_off + 2 * (groups + 1);
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
  const int n0 = static_cast<int>(local) * BN;
  const int nk = (K + BK - 1) / BK;
  int k_lo = nk * ks / split * BK, k_hi = min(K, nk * (ks + 1) / split * BK);
  const bf16_t* Bk;
  if constexpr (BKN) {  // B [K][N], rows k_lo.. of B0, or all of B0 / B1 for the two halves
    if (B1 != nullptr) {
      k_lo = ks * (K / 2);
      k_hi = k_lo + K / 2;
      Bk = ks == 0 ? B0 : B1;
    } else {
      Bk = B0 + static_cast<int64_t>(k_lo) * N;
    }
  } else {
    Bk = B0 + k_lo;
  }
  // the tile's rows start at row 0 of the partial block: A (or the gather list) moves instead
  const bf16_t* Ak = GATHER ? A + k_lo : A + static_cast<int64_t>(row_begin) * K + k_lo;
  const int32_t* gk = GATHER ? gather + row_begin : nullptr;
  bf16_t* P = reinterpret_cast<bf16_t*>(part + (static_cast<int64_t>(ks) * groups + g) * 128 * N);
  if (table == t128)
    run_tile<2, KTAIL, GATHER, 128, BKN>(lds, Ak, K, gk, Bk, nullptr, group_stride, BKN ? N : K, N,
                                         k_hi - k_lo, P, N, nullptr, nullptr, g, 0, rows, n0);
  else
    run_tile<2, KTAIL, GATHER, 64, BKN>(lds, Ak, K, gk, Bk, nullptr, group_stride, BKN ? N : K, N,
                                        k_hi - k_lo, P, N, nullptr, nullptr, g, 0, rows, n0);
}

// tile_off: three tables of groups + 1 entries: 256-row tiles, 128-row tiles, 64-row tiles.
// Blocks [0, main_blocks) serve the 256-row tiles, the rest the smaller ones.
template <int EPI, bool KTAIL, bool GATHER, bool BKN = false>
__global__ __launch_bounds__(NT, 1) void grouped_gemm_kernel(
    const bf16_t* __restrict__ A, const int32_t* __restrict__ gather,
    const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ tile_off, int groups, int main_blocks,
    const bf16_t* __restrict__ B0, const bf16_t* __restrict__ B1, int64_t group_stride, int N,
    int K, bf16_t* __restrict__ C, float* __restrict__ C2, float* __restrict__ C3,
    float* __restrict__ part, int split) {
  constexpr int BNO = (EPI == 0 || EPI == 3 || EPI == 4) ? BN / 2 : BN;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int nb_count = (N + BNO - 1) / BNO;
  const int32_t* t256 = tile_off;
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
  if constexpr ((EPI == 1 && !GATHER && !BKN) || (EPI == 2 && BKN)) {
    if (split > 1) {  // remainder tiles in K chunks: fp32 partials, summed by finish_split_kernel
      const int64_t Lr = static_cast<int64_t>(blockIdx.x) - main_blocks;
      run_remainder_split<EPI, KTAIL, GATHER, BKN>(lds, Lr / split, static_cast<int>(Lr % split),
                                                   split, A, gather, offsets, tile_off, groups, B0,
                                                   B1, group_stride, N, K, part);
      return;
    }
  }
  run_remainder_tile<EPI, KTAIL, GATHER, BKN>(lds, static_cast<int64_t>(blockIdx.x) - main_blocks,
                                             A, gather, offsets, tile_off, groups, B0, B1,
                                             group_stride, N, K, C, C2, C3);
}

// The rows of the split remainder tiles: out row = the sum over the K chunks, in chunk order, of
// the fp32 partials (rounded once to bf16, or fp32 with OUT_F32), for each group's 1..128 rows
// past its 256-row tiles. One block per (group, remainder row), 8 columns per thread.
template <bool OUT_F32>
__global__ __launch_bounds__(256) void finish_split_kernel(const int32_t* __restrict__ offsets,
                                                           int groups, int N, int split,
                                                           const float* __restrict__ part,
                                                           bf16_t* __restrict__ out) {
  const int g = static_cast<int>(blockIdx.x) / 128, r = static_cast<int>(blockIdx.x) % 128;
  const int rows_g = offsets[g + 1] - offsets[g];
  const int rem = rows_g & 255;
  if (rem == 0 || rem > 128 || r >= rem) return;
  const int c = (static_cast<int>(blockIdx.y) * 256 + static_cast<int>(threadIdx.x)) * 8;
  if (c >= N) return;
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = 0.f;
  for (int ks = 0; ks < split; ++ks) {
    const float* p = part + ((static_cast<int64_t>(ks) * groups + g) * 128 + r) * N + c;
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] += a.x; v[1] += a.y; v[2] += a.z; v[3] += a.w;
    v[4] += b.x; v[5] += b.y; v[6] += b.z; v[7] += b.w;
  }
  const int64_t row = offsets[g] + (rows_g & ~255) + r;
  if constexpr (OUT_F32) {
    float* o = reinterpret_cast<float*>(out) + row * N + c;
    *reinterpret_cast<float4*>(o) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(o + 4) = make_float4(v[4], v[5], v[6], v[7]);
  } else {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = static_cast<uint32_t>(f32_to_bf16(v[2 * i])) |
             (static_cast<uint32_t>(f32_to_bf16(v[2 * i + 1])) << 16);
    *reinterpret_cast<uint4*>(out + row * N + c) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// One grouped product of the persistent kernel: groups of rows [offsets[g], offsets[g+1]) of A
// (row r is A[gather[r]] when gather is set), weights B0 (and B1 for the paired gate/up columns)
// at group_stride per group, N output columns, reduction K, output C [rows][N].
struct GemmProb {
  const bf16_t* A;
  const int32_t* gather;
  const int32_t* offsets;
  const int32_t* tile_off;  // three tile tables of groups + 1 entries
  const bf16_t* B0;
  const bf16_t* B1;
  int64_t group_stride;
  bf16_t* C;
  int groups, N, K;
  float* C2;  // EPI 3: U (C holds G as floats)
  float* C3;
};

// Persistent form of the products with bf16 or fp32 row outputs (EPI 0: SwiGLU to bf16 h; EPI 1:
// plain bf16; EPI 3: the fp32 gate and up pre-activations) for K of 2..128 k-slices, over the 256-row tiles of one or two products (the routed experts, and the
// shared experts as a second product of one group). Each XCD x owns the tiles [x q_p, (x+1) q_p)
// of each product p (the second product's first: its tiles are the longer ones when K differs);
// slot s of its S blocks takes entries s, s + S, ... of that list, and the k-step pipeline runs on
// across tiles: the last two k-steps of a tile load the first two k-slices of the block's next
// tile, the last one stores the first of them and reads its first fragments, so the next tile's
// MFMAs start right after this tile's epilogue with no memory round trip, tile lookup or block
// launch in between. The next tile's product, group, rows and A-row offsets are looked up at the
// start of the current tile. The epilogue goes through the LDS stage the tile's last k-step read;
// the other stage holds the next tile's first slice.
template <int EPI, bool KTAIL, bool GATHER>
__device__ __forceinline__ void run_tiles_persistent(unsigned char* lds, const GemmProb& P0,
                                                     const GemmProb& P1, int nblocks) {
  static_assert(EPI == 0 || EPI == 1 || EPI == 3, "persistent epilogues");
  using G = Geo<256>;
  constexpr bool PAIRED = EPI != 1, SWIGLU = EPI == 0 || EPI == 4;
  constexpr bool F32PAIR = EPI == 3;  // fp32 gate and up pre-activations out
  constexpr int BNO = PAIRED ? BN / 2 : BN;
  constexpr int MI = G::MI, NJ = G::NJ, ACH = G::ACH, BCH = G::BCH, RS = G::RSTEP;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / G::WN, wn = wave % G::WN;

  const int nb0 = (P0.N + BNO - 1) / BNO;
  const int nb1 = P1.groups > 0 ? (P1.N + BNO - 1) / BNO : 0;
  const int64_t nt0 = static_cast<int64_t>(P0.tile_off[P0.groups]) * nb0;
  const int64_t nt1 = P1.groups > 0 ? static_cast<int64_t>(P1.tile_off[P1.groups]) * nb1 : 0;
  const int64_t q0 = (nt0 + NXCD - 1) / NXCD, q1 = (nt1 + NXCD - 1) / NXCD;
  const int S = nblocks / NXCD;
  const int xcd = static_cast<int>(blockIdx.x) % NXCD, slot = static_cast<int>(blockIdx.x) / NXCD;
  const int64_t b1 = static_cast<int64_t>(xcd) * q1, b0 = static_cast<int64_t>(xcd) * q0;
  const int64_t n1x = max(int64_t{0}, min(b1 + q1, nt1) - b1);
  const int64_t n0x = max(int64_t{0}, min(b0 + q0, nt0) - b0);
  const int64_t xend = n1x + n0x;  // entries of this XCD's list
  int64_t J = slot;
  if (J >= xend) return;

  struct Tile {
    int p, g, row_begin, rows, n0;
  };
  auto describe = [&](int64_t Jt) __attribute__((always_inline)) {
    Tile t;
    t.p = Jt < n1x ? 1 : 0;
    const GemmProb& P = t.p ? P1 : P0;
    const int nb = t.p ? nb1 : nb0;
    const int64_t Lt = t.p ? b1 + Jt : b0 + (Jt - n1x);
    t.g = find_group(P.tile_off, P.groups, nb, Lt);
    const int mt_g = P.tile_off[t.g + 1] - P.tile_off[t.g];
    const int64_t local = Lt - static_cast<int64_t>(P.tile_off[t.g]) * nb;
    const int nbi = static_cast<int>(local / mt_g), mt = static_cast<int>(local % mt_g);
    t.row_begin = P.offsets[t.g] + mt * 256;
    t.rows = min(256, P.offsets[t.g + 1] - t.row_begin);
    t.n0 = nbi * BNO;
    return t;
  };

  // ---- load addressing of the tile whose k-slices are being loaded (as in run_tile, with every
  // A row as a 32-bit byte offset from its A: the launcher checks that each A spans < 4 GiB)
  const int r0 = tid >> 3, kc_t = (tid & 7) * 8;
  const char* a_base = nullptr;
  int ldK = 0;  // K (and the row stride of A and B) of that tile
  uint32_t a_off[ACH], b_off[BCH];
  const char* b_base0 = nullptr;
  const char* b_base1 = nullptr;
  uint32_t gn[ACH];  // byte offsets of this thread's A rows in the next tile (gathered or not)
  auto fetch_gather = [&](const Tile& t) __attribute__((always_inline)) {
    const GemmProb& P = t.p ? P1 : P0;
    const int32_t* gth = (GATHER && t.p == 0) ? P0.gather : nullptr;
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int r = t.row_begin + min(i * RS + r0, t.rows - 1);
      gn[i] = static_cast<uint32_t>(gth != nullptr ? gth[r] : r) * static_cast<uint32_t>(P.K * 2) +
              static_cast<uint32_t>(kc_t * 2);
    }
  };
  auto set_ld = [&](const Tile& t) __attribute__((always_inline)) {
    const GemmProb& P = t.p ? P1 : P0;
#pragma unroll
    for (int i = 0; i < ACH; ++i) a_off[i] = gn[i];
    a_base = reinterpret_cast<const char*>(P.A);
    ldK = P.K;
    const bf16_t* Bg0 =
        P.B0 + static_cast<int64_t>(t.g) * P.group_stride + static_cast<int64_t>(t.n0) * P.K;
    const bf16_t* Bg1 = PAIRED ? P.B1 + static_cast<int64_t>(t.g) * P.group_stride +
                                     static_cast<int64_t>(t.n0) * P.K
                               : Bg0;
    b_base0 = reinterpret_cast<const char*>(Bg0);
    b_base1 = reinterpret_cast<const char*>(Bg1);
    const int b_rows = min(PAIRED ? BN / 2 : BN, P.N - t.n0);
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
      const int r = i * RS + r0;
      const int rb_ = PAIRED ? (r & (BN / 2 - 1)) : r;
      b_off[i] = static_cast<uint32_t>((min(rb_, b_rows - 1) * P.K + kc_t) * 2);
    }
  };
  u32x4 ra[ACH], rb[BCH];
  auto gload = [&](int k0) __attribute__((always_inline)) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
    const bool in = !KTAIL || k0 + kc_t < ldK;
    const uint32_t kb = static_cast<uint32_t>((in ? k0 : ldK - 8 - kc_t) * 2);
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(a_base + (a_off[i] + kb));
      ra[i] = KTAIL ? (in ? v : zero) : v;
    }
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
      const char* bb = (PAIRED && i >= BCH / 2) ? b_base1 : b_base0;
      const u32x4 v = *reinterpret_cast<const u32x4*>(bb + (b_off[i] + kb));
      rb[i] = KTAIL ? (in ? v : zero) : v;
    }
  };
  const uint32_t st_off = static_cast<uint32_t>(swz(r0, tid & 7) * 2);
  constexpr uint32_t kStageBytes = G::STAGE, kBBytes = 256 * BK * 2;
  auto lstore = [&](int stage) __attribute__((always_inline)) {
    unsigned char* sa = lds + stage * kStageBytes + st_off;
#pragma unroll
    for (int i = 0; i < ACH; ++i) *reinterpret_cast<u32x4*>(sa + i * RS * BK * 2) = ra[i];
#pragma unroll
    for (int i = 0; i < BCH; ++i)
      *reinterpret_cast<u32x4*>(sa + kBBytes + i * RS * BK * 2) = rb[i];
  };

  f32x16 acc[MI][NJ];
  const int l32 = lane & 31, lk = lane >> 5, sw = (l32 >> 1) & 7;
  uint32_t fo[4];
#pragma unroll
  for (int sub = 0; sub < 4; ++sub)
    fo[sub] = static_cast<uint32_t>((l32 * BK + (((sub * 2 + lk) ^ sw) << 3)) * 2);
  int brow[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j)
    brow[j] = PAIRED ? ((j < NJ / 2 ? 0 : BN / 2) + wn * (G::WCOLS / 2) + (j % (NJ / 2)) * 32)
                     : (wn * G::WCOLS + j * 32);
  bf16x8 fa[2][MI], fb[2][NJ];
  auto lfrag = [&](int set, int stage, int sub) __attribute__((always_inline)) {
    const unsigned char* sa = lds + stage * kStageBytes + fo[sub];
#pragma unroll
    for (int i = 0; i < MI; ++i)
      fa[set][i] = *reinterpret_cast<const bf16x8*>(sa + (wm * G::WROWS + i * 32) * BK * 2);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      fb[set][j] = *reinterpret_cast<const bf16x8*>(sa + kBBytes + brow[j] * BK * 2);
  };
  // MFMA order: the B fragment runs backwards on odd row blocks, so consecutive MFMAs share an
  // operand across the row-block boundary too (fewer operand bits switch: a power-limited clock)
  auto mfmas = [&](int set) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) {
        const int j = (i & 1) ? NJ - 1 - jj : jj;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[set][i], fb[set][j], acc[i][j], 0, 0, 0);
      }
  };
  constexpr int NMF = MI * NJ, NR = MI + NJ, NX = ACH + BCH;
  // one k-step on stage `cur`, with the same sub-step schedule as run_tile; the slice stored and
  // the one loaded are the next two of the block's slice stream, of this tile or the next
  auto kstep = [&](int cur, int k0) __attribute__((always_inline)) {
    lfrag(1, cur, 1);
    mfmas(0);
    lstore(cur ^ 1);
    gload(k0);
    sched_substep_wl<NMF, NR, NX, NX>();
    lfrag(0, cur, 2);
    mfmas(1);
    sched_substep<NMF, NR, 0, 0>();
    lfrag(1, cur, 3);
    mfmas(0);
    sched_substep<NMF, NR, 0, 0>();
    __syncthreads();
    lfrag(0, cur ^ 1, 0);
    mfmas(1);
    sched_substep<NMF, NR, 0, 0>();
  };
  // Epilogue through LDS: each wave writes its outputs as bf16 into a private 8 KB region of the
  // stage the tile's last k-step read (free once that k-step's barrier has passed), reads them
  // back as 16-byte row chunks and stores those; SwiGLU tiles take one pass (128 rows x 32
  // columns per wave), plain tiles two (64 rows x 64 columns). Row chunks are XOR-swizzled by row.
  // A barrier follows, before the next tile's first k-step stores into that stage. The lane's row
  // and column pass through an empty asm statement, so that its LDS offsets are formed here, tile
  // by tile, rather than hoisted out of the tile loop into registers.
  constexpr int PC = SWIGLU ? 32 : 64;          // columns of a wave's bf16 pass
  constexpr int PR = 4096 / PC;                 // rows of a pass (8 KB of bf16)
  constexpr int PCH = PC / 8;                   // 16-byte chunks per row
  constexpr int PI = PR / 32;                   // 32-row blocks per pass
  auto epilogue = [&](const Tile& t, int free_stage) __attribute__((always_inline)) {
    const GemmProb& P = t.p ? P1 : P0;
    bf16_t* C = P.C;
    const int N = P.N, ldc = P.N;
    unsigned char* reg = lds + free_stage * kStageBytes + wave * 8192;
    const bool full = t.rows == 256 && t.n0 + BNO <= N;
    int lrow = lk * 4, lcol = l32, ln = lane;
    asm volatile("" : "+v"(lrow), "+v"(lcol), "+v"(ln));
    if constexpr (F32PAIR) {
      // fp32 G (accumulators jj) then U (jj + NJ / 2), 64 rows x 32 columns per pass: row r of
      // the region at byte (128 r) ^ 128 ((r >> 2) & 1), so that the half-waves of a store (rows
      // 4 apart) use different banks; 8 chunks of 16 bytes per row on the way out
      static_assert(NJ / 2 == 1 && MI % 2 == 0, "one 32-column block per wave and operand");
      float* Cg = reinterpret_cast<float*>(P.C);
      float* Cu = P.C2;
#pragma unroll
      for (int i0 = 0; i0 < MI; i0 += 2)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
#pragma unroll
          for (int ii = 0; ii < 2; ++ii)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int row = ii * 32 + (r >> 2) * 8 + lrow + (r & 3);
              *reinterpret_cast<float*>(reg + ((row * 128) ^ (((row >> 2) & 1) << 7)) + lcol * 4) =
                  acc[i0 + ii][q * (NJ / 2)][r];
            }
          float* Co = q ? Cu : Cg;
#pragma unroll
          for (int qq = 0; qq < 8; ++qq) {
            const int idx = qq * 64 + ln, rr = idx >> 3, c = idx & 7;
            const u32x4 v =
                *reinterpret_cast<const u32x4*>(reg + ((rr * 128) ^ (((rr >> 2) & 1) << 7)) + c * 16);
            const int row = wm * G::WROWS + i0 * 32 + rr;
            const int col = t.n0 + wn * (G::WCOLS / 2) + c * 4;
            if (full || (row < t.rows && col < N))
              __builtin_nontemporal_store(
                  v, reinterpret_cast<u32x4*>(Co + static_cast<int64_t>(t.row_begin + row) * ldc + col));
          }
        }
    }
#pragma unroll
    for (int i0 = 0; i0 < (EPI == 3 ? 0 : MI); i0 += PI) {
#pragma unroll
      for (int i = i0; i < i0 + PI; ++i)
#pragma unroll
        for (int jj = 0; jj < (SWIGLU ? NJ / 2 : NJ); ++jj)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = (i - i0) * 32 + (r >> 2) * 8 + lrow + (r & 3);
            const int col = jj * 32 + lcol;
            const float v = SWIGLU ? silu(acc[i][jj][r]) * acc[i][jj + NJ / 2][r] : acc[i][jj][r];
            *reinterpret_cast<bf16_t*>(reg + row * (PC * 2) + (((col >> 3) ^ (row & (PCH - 1))) << 4) +
                                       (col & 7) * 2) = f32_to_bf16(v);
          }
#pragma unroll
      for (int qq = 0; qq < (PR * PCH) / 64; ++qq) {
        const int idx = qq * 64 + ln, rr = idx / PCH, c = idx % PCH;
        const u32x4 v = *reinterpret_cast<const u32x4*>(reg + rr * (PC * 2) + ((c ^ (rr & (PCH - 1))) << 4));
        const int row = wm * G::WROWS + i0 * 32 + rr;
        const int col = t.n0 + (SWIGLU ? wn * (G::WCOLS / 2) : wn * G::WCOLS) + c * 8;
        if (full || (row < t.rows && col < N))
          __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(C + static_cast<int64_t>(t.row_begin + row) * ldc + col));
      }
    }
    __syncthreads();
  };

  Tile cur = describe(J);
  fetch_gather(cur);
  set_ld(cur);
  gload(0);
  lstore(0);
  gload(BK);
  __syncthreads();
  lfrag(0, 0, 0);
  int sb = 0;  // stage of the tile's first k-slice
  for (;;) {
    const int64_t Jn = J + S;
    const bool has_next = Jn < xend;
    Tile nxt = cur;
    if (has_next) {
      nxt = describe(Jn);
      fetch_gather(nxt);
    }
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    const int nk = ((cur.p ? P1.K : P0.K) + BK - 1) / BK;  // >= 2
    // the last two k-steps load the next tile's first two slices (the block's last tile loads its
    // own again, unused)
    for (int kt = 0; kt < nk; ++kt) {
      if (kt == nk - 2) set_ld(nxt);
      const int k0 = (kt + 2 < nk ? kt + 2 : kt + 2 - nk) * BK;
      kstep((sb + kt) & 1, k0);
    }
    epilogue(cur, (sb + nk - 1) & 1);
    if (!has_next) break;
    sb ^= nk & 1;
    cur = nxt;
    J = Jn;
  }
  // the last tile's final two k-steps re-read its own first slices; let them land before exit
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Blocks [0, main_blocks) run the persistent tile lists; the rest run the remainder tiles of the
// first product, then of the second (at most one 128-row and one 64-row tile per group).
template <int EPI, bool KTAIL, bool GATHER>
__global__ __launch_bounds__(NT, 1) void grouped_gemm_persistent_kernel(GemmProb P0, GemmProb P1,
                                                                        int main_blocks) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  if (static_cast<int>(blockIdx.x) < main_blocks) {
    run_tiles_persistent<EPI, KTAIL, GATHER>(lds, P0, P1, main_blocks);
    return;
  }
  constexpr int BNO = EPI != 1 ? BN / 2 : BN;
  int64_t L = static_cast<int64_t>(blockIdx.x) - main_blocks;
  const int64_t r0 = 2 * static_cast<int64_t>(P0.groups) * ((P0.N + BNO - 1) / BNO);
  if (L < r0) {
    run_remainder_tile<EPI, KTAIL, GATHER, false>(lds, L, P0.A, P0.gather, P0.offsets,
                                                  P0.tile_off, P0.groups, P0.B0, P0.B1,
                                                  P0.group_stride, P0.N, P0.K, P0.C, P0.C2,
                                                  P0.C3);
    return;
  }
  if (P1.groups > 0)
    run_remainder_tile<EPI, KTAIL, false, false>(lds, L - r0, P1.A, nullptr, P1.offsets,
                                                 P1.tile_off, P1.groups, P1.B0, P1.B1,
                                                 P1.group_stride, P1.N, P1.K, P1.C, P1.C2,
                                                 P1.C3);
}

// Weight gradients, with both operands read in place K-major: C_g [Ma][Nb] (fp32) = sum over the
// rows r of group g, [offsets[g], offsets[g+1]), of A[r][m] B[r][n], for row-major A [rows][lda]
// and B [rows][ldb] (the rows of all groups, `rows` in total). Persistent, as the forward
// products: one block per CU walks its XCD's run of the tile list (256 x 256 output tiles of each
// group in bands of 8 m-tiles, n fastest in a band, so that concurrent tiles share operand slabs;
// the XCDs split the list by k-steps, as the groups' row counts differ), and the last two k-steps
// of a tile load the next tile's first two k-slices. A k-slice is 64 rows of the tile's 256 A
// columns and 256 B columns, staged as two [64 k][256] LDS slices (512-byte rows, 16-byte chunks
// XOR-swizzled by 64 bytes); rows past the group's end are stored as zeros, and both MFMA operands
// come from transposing LDS reads (ds_read_b64_tr_b16). A group spans kt[g+1] - kt[g] >= 2
// k-slices (the schedule gives short and empty groups zero slices), so every tile has the two
// k-steps that hand over to the next. The fp32 tile leaves through the free LDS stage: each wave
// stages 32 x 64 floats of its 128 x 64 block at a time in a private 8 KB region and stores them
// as 16-byte row pieces (32 stores per lane), so the next tile's loads can be waited on while those
// stores are still in flight.
__device__ __forceinline__ void run_wgrad_persistent(unsigned char* lds,
                                                     const bf16_t* __restrict__ A, int lda,
                                                     const bf16_t* __restrict__ B, int ldb,
                                                     int rows, const int32_t* __restrict__ offsets,
                                                     const int32_t* __restrict__ kt, int groups,
                                                     int Ma, int Nb, float* __restrict__ C,
                                                     int nblocks) {
  using G = Geo<256>;
  constexpr int MI = G::MI, NJ = G::NJ;
  static_assert(NT == 512 && G::WCOLS == 64 && MI * 32 == G::WROWS, "wave layout of the tiles");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / G::WN, wn = wave % G::WN;
  const int mt = (Ma + 255) / 256, nt = (Nb + 255) / 256;
  const int64_t per_group = static_cast<int64_t>(mt) * nt;
  const int S = nblocks / NXCD;
  const int xcd = static_cast<int>(blockIdx.x) % NXCD, slot = static_cast<int>(blockIdx.x) / NXCD;
  // the XCDs split the list by work: the tiles before tile L (group g, local index l) hold
  // per_group kt[g] + l (kt[g+1] - kt[g]) k-steps, and XCD x takes the tiles that start in
  // [x W / 8, (x + 1) W / 8) of the total W
  auto first_tile = [&](int64_t work) __attribute__((always_inline)) {
    int lo = 0, hi = groups;  // largest g with per_group kt[g] <= work
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (per_group * kt[mid] <= work) lo = mid; else hi = mid;
    }
    const int64_t nk = kt[lo + 1] - kt[lo];  // >= 2
    const int64_t l = min(per_group, (work - per_group * kt[lo] + nk - 1) / nk);
    return static_cast<int64_t>(lo) * per_group + l;
  };
  const int64_t W = per_group * kt[groups];
  const int64_t b0 = first_tile(W * xcd / NXCD);
  const int64_t xend = first_tile(W * (xcd + 1) / NXCD) - b0;
  int64_t J = slot;
  if (J >= xend) return;

  struct Tile {
    int g, m0, n0, r_lo, r_hi, nk;
  };
  constexpr int kWgBand = 8;
  auto describe = [&](int64_t Jt) __attribute__((always_inline)) {
    Tile t;
    const int64_t L = b0 + Jt;
    t.g = static_cast<int>(L / per_group);
    const int local = static_cast<int>(L % per_group);
    const int band = local / (kWgBand * nt), w = local % (kWgBand * nt);
    const int bw = min(kWgBand, mt - band * kWgBand);
    t.m0 = (band * kWgBand + w % bw) * 256;
    t.n0 = (w / bw) * 256;
    t.r_lo = offsets[t.g];
    t.r_hi = offsets[t.g + 1];
    t.nk = kt[t.g + 1] - kt[t.g];  // >= 2
    return t;
  };

  // ---- loads: thread tid moves the 16-byte chunk (tid % 32) of rows 16 i + tid / 32 (i < 4) of
  // both slices. Columns past Ma or Nb re-read the last 8 (they only reach outputs never stored);
  // a row past the group reads a valid row and is stored as zeros.
  const int krow = tid >> 5, kc = tid & 31;
  const char* a_col = nullptr;
  const char* b_col = nullptr;
  int64_t r_base = 0, r_end = 0;  // first row of the loading tile's group, and its end
  auto set_ld = [&](const Tile& t) __attribute__((always_inline)) {
    a_col = reinterpret_cast<const char*>(A + min(t.m0 + kc * 8, Ma - 8));
    b_col = reinterpret_cast<const char*>(B + min(t.n0 + kc * 8, Nb - 8));
    r_base = t.r_lo + krow;
    r_end = t.r_hi;
  };
  u32x4 ra[4], rb[4];
  uint32_t live = 0;  // bit i: row 16 i + krow of the slice belongs to the group
  auto gload = [&](int k0) __attribute__((always_inline)) {
    live = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t r = r_base + k0 + 16 * i;
      live |= (r < r_end ? 1u : 0u) << i;
      const int64_t rr = r < rows ? r : rows - 1;
      ra[i] = *reinterpret_cast<const u32x4*>(a_col + rr * lda * 2);
      rb[i] = *reinterpret_cast<const u32x4*>(b_col + rr * ldb * 2);
    }
  };
  // LDS: [64 k][256] slices of 512-byte rows, chunk c of row r at chunk c ^ 4 (r & 3); a thread's
  // rows are 16 apart, so r & 3 is the same for all of them
  constexpr uint32_t kStageBytes = G::STAGE, kBBytes = 256 * BK * 2;
  const uint32_t st_off = static_cast<uint32_t>(krow * 512 + ((kc ^ ((krow & 3) << 2)) << 4));
  auto lstore = [&](int stage) __attribute__((always_inline)) {
    unsigned char* sa = lds + stage * kStageBytes + st_off;
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool in = (live >> i) & 1u;
      *reinterpret_cast<u32x4*>(sa + i * 16 * 512) = in ? ra[i] : zero;
      *reinterpret_cast<u32x4*>(sa + kBBytes + i * 16 * 512) = in ? rb[i] : zero;
    }
  };

  // ---- fragments by transposing reads: in each group of 16 lanes, lane 4 q + a reads 4 columns
  // (c_base + 4 a ..) of row k_base + q, and lane i receives rows k_base .. k_base + 3 of column
  // c_base + i. Lane l's 32x32x16 operand (8 k of row or column l % 32) is two such reads, rows
  // 16 sub + 8 (l / 32) + {0..3} and {4..7}; the A operand (rows m of C) reads the A slice the same
  // way the B operand reads the B slice.
  f32x16 acc[MI][NJ];
  const int g4 = lane >> 4, i16 = lane & 15;
  const int trow = 8 * (g4 >> 1) + (i16 >> 2);
  auto tr_off = [&](int col) {
    return static_cast<uint32_t>(trow * 512 + (((col >> 3) ^ ((i16 >> 2) << 2)) << 4) +
                                 (((col >> 2) & 1) << 3));
  };
  uint32_t ta_off[MI], tb_off[NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i) ta_off[i] = tr_off(wm * G::WROWS + i * 32 + 16 * (g4 & 1) + 4 * (i16 & 3));
#pragma unroll
  for (int j = 0; j < NJ; ++j)
    tb_off[j] = kBBytes + tr_off(wn * G::WCOLS + j * 32 + 16 * (g4 & 1) + 4 * (i16 & 3));
  bf16x8 fa[2][MI], fb[2][NJ];
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  auto trpair = [&](const unsigned char* p) __attribute__((always_inline)) {
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p + 4 * 512));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto lfrag = [&](int set, int stage, int sub) __attribute__((always_inline)) {
    const unsigned char* sb = lds + stage * kStageBytes + sub * 16 * 512;
#pragma unroll
    for (int i = 0; i < MI; ++i) fa[set][i] = trpair(sb + ta_off[i]);
#pragma unroll
    for (int j = 0; j < NJ; ++j) fb[set][j] = trpair(sb + tb_off[j]);
  };
  // MFMA order: the B fragment runs backwards on odd row blocks, so consecutive MFMAs share an
  // operand across the row-block boundary too (fewer operand bits switch: a power-limited clock)
  auto mfmas = [&](int set) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) {
        const int j = (i & 1) ? NJ - 1 - jj : jj;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[set][i], fb[set][j], acc[i][j], 0, 0, 0);
      }
  };
  constexpr int NMF = MI * NJ, NR = 2 * (MI + NJ), NX = 8;
  auto kstep = [&](int cur, int k0) __attribute__((always_inline)) {
    lfrag(1, cur, 1);
    mfmas(0);
    lstore(cur ^ 1);
    gload(k0);
    sched_substep_wl<NMF, NR, NX, NX>();
    lfrag(0, cur, 2);
    mfmas(1);
    sched_substep<NMF, NR, 0, 0>();
    lfrag(1, cur, 3);
    mfmas(0);
    sched_substep<NMF, NR, 0, 0>();
    __syncthreads();
    lfrag(0, cur ^ 1, 0);
    mfmas(1);
    sched_substep<NMF, NR, 0, 0>();
  };
  // Epilogue: pass i stages the wave's rows 32 i .. 32 i + 31 (64 columns) as fp32 in its 8 KB
  // region, 16-byte chunk c of row r at chunk c ^ 8 ((r >> 2) & 1) (a store instruction's two
  // half-waves write rows 4 apart, which then fall on different banks), and stores them as 16
  // chunks per row. A barrier follows before the next tile's first k-step stores into the stage.
  auto epilogue = [&](const Tile& t, int free_stage) __attribute__((always_inline)) {
    float* Cg = C + static_cast<int64_t>(t.g) * Ma * Nb;
    unsigned char* reg = lds + free_stage * kStageBytes + wave * 8192;
    const int orows = min(256, Ma - t.m0), ocols = min(256, Nb - t.n0);
    const bool full = orows == 256 && ocols == 256;
    const int l32 = lane & 31, lk = lane >> 5;
    int lrow = lk * 4, lcol = l32, ln = lane;
    asm volatile("" : "+v"(lrow), "+v"(lcol), "+v"(ln));
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = (r >> 2) * 8 + lrow + (r & 3);
          const int col = j * 32 + lcol;
          *reinterpret_cast<float*>(reg + row * 256 + (((col >> 2) ^ (((row >> 2) & 1) << 3)) << 4) +
                                    (col & 3) * 4) = acc[i][j][r];
        }
#pragma unroll
      for (int qq = 0; qq < 8; ++qq) {
        const int idx = qq * 64 + ln, rr = idx >> 4, c = idx & 15;
        const u32x4 v =
            *reinterpret_cast<const u32x4*>(reg + rr * 256 + ((c ^ (((rr >> 2) & 1) << 3)) << 4));
        const int row = wm * G::WROWS + i * 32 + rr;
        const int col = wn * G::WCOLS + c * 4;
        if (full || (row < orows && col < ocols))
          __builtin_nontemporal_store(
              v, reinterpret_cast<u32x4*>(Cg + static_cast<int64_t>(t.m0 + row) * Nb + t.n0 + col));
      }
    }
    __syncthreads();
  };

  Tile cur = describe(J);
  set_ld(cur);
  gload(0);
  lstore(0);
  gload(BK);
  __syncthreads();
  lfrag(0, 0, 0);
  int sb = 0;  // stage of the tile's first k-slice
  for (;;) {
    const int64_t Jn = J + S;
    const bool has_next = Jn < xend;
    const Tile nxt = has_next ? describe(Jn) : cur;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    const int nk = cur.nk;
    for (int k = 0; k < nk; ++k) {
      if (k == nk - 2) set_ld(nxt);
      const int k0 = (k + 2 < nk ? k + 2 : k + 2 - nk) * BK;
      kstep((sb + k) & 1, k0);
    }
    epilogue(cur, (sb + nk - 1) & 1);
    if (!has_next) break;
    sb ^= nk & 1;
    cur = nxt;
    J = Jn;
  }
  // the last tile's final two k-steps re-read its own first slices; let them land before exit
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

__global__ __launch_bounds__(NT, 1) void wgrad_persistent_kernel(
    const bf16_t* __restrict__ A, int lda, const bf16_t* __restrict__ B, int ldb, int rows,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ kt, int groups, int Ma,
    int Nb, float* __restrict__ C) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  run_wgrad_persistent(lds, A, lda, B, ldb, rows, offsets, kt, groups, Ma, Nb, C,
                       static_cast<int>(gridDim.x));
}

// Compute units of the current device, rounded down to a multiple of the XCD count (0 if unknown).
int persistent_blocks() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    v = cus / NXCD * NXCD;
    cached[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

// Whether the persistent kernel serves a forward product: 2..128 k-slices (long-K tiles keep the
// one-tile blocks: their per-tile costs are small, and the persistent loop measured ~2% slower per
// k-step on the 224-step down projection of the Mixtral layer), A (a_rows rows of K) spanning less
// than 4 GiB (32-bit row offsets), and a known compute-unit count.
bool persistent_ok(const GemmProb& P, int64_t a_rows) {
  return P.K >= 2 * BK && P.K <= 128 * BK && a_rows >= 0 &&
         a_rows * P.K * 2 < (int64_t{1} << 32) && persistent_blocks() >= NXCD;
}

// One launch of the persistent kernel over one product (P1.groups == 0) or two.
template <int EPI, bool KTAIL, bool GATHER>
hipError_t launch_persistent(const GemmProb& P0, int64_t max_tiles0, const GemmProb& P1,
                             int64_t max_tiles1, hipStream_t st) {
  constexpr int BNO = EPI != 1 ? BN / 2 : BN;
  constexpr size_t kMainP = 2 * Geo<256>::STAGE;
  constexpr size_t kEpiR = static_cast<size_t>(128) * (BNO + 8) * sizeof(bf16_t);
  constexpr size_t ldsp = kMainP > kEpiR ? kMainP : kEpiR;
  static std::atomic<bool> attr_p{false};
  if (!attr_p.load(std::memory_order_acquire)) {
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&grouped_gemm_persistent_kernel<EPI, KTAIL, GATHER>),
        hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(ldsp));
    if (e != hipSuccess) return e;
    attr_p.store(true, std::memory_order_release);
  }
  const int64_t nb0 = cdiv(P0.N, BNO), nb1 = P1.groups > 0 ? cdiv(P1.N, BNO) : 0;
  const int64_t tiles = max_tiles0 * nb0 + (P1.groups > 0 ? max_tiles1 * nb1 : 0);
  if (tiles <= 0) return hipSuccess;
  const int64_t pb = persistent_blocks();
  const int64_t upper = cdiv(tiles, NXCD) * NXCD;
  const int64_t main_blocks = upper < pb ? upper : pb;
  const int64_t grid = main_blocks + 2 * static_cast<int64_t>(P0.groups) * nb0 +
                       2 * static_cast<int64_t>(P1.groups) * nb1;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((grouped_gemm_persistent_kernel<EPI, KTAIL, GATHER>),
                     dim3(static_cast<unsigned>(grid)), dim3(NT), ldsp, st, P0, P1,
                     static_cast<int>(main_blocks));
  return hipGetLastError();
}

template <int EPI, bool KTAIL, bool GATHER, bool BKN = false>
hipError_t launch_gemm_t(const bf16_t* A, const int32_t* gather, const int32_t* offsets,
                         const int32_t* tile_off,
                         int groups, int64_t max_tiles, const bf16_t* B0, const bf16_t* B1,
                         int64_t group_stride, int N, int K, bf16_t* C, float* C2,
                         float* C3, hipStream_t st, int64_t a_rows, float* part) {
  constexpr int BNO = (EPI == 0 || EPI == 3 || EPI == 4) ? BN / 2 : BN;
  const int64_t nb = cdiv(N, BNO);
  // (the training forward's EPI 4 stays one tile per block: its persistent form spills registers)
  if constexpr ((EPI == 0 || EPI == 1 || EPI == 3) && !BKN) {
    GemmProb P0{A, gather, offsets, tile_off, B0, B1, group_stride, C, groups, N, K, C2, C3};
    GemmProb none{};
    if (persistent_ok(P0, a_rows))
      return launch_persistent<EPI, KTAIL, GATHER>(P0, max_tiles, none, 0, st);
  }
  // the remainder tiles of a plain long-K product in two K chunks, so that they spread over all
  // CUs instead of running as a short last round on a few (part: [2][groups][128][N] fp32)
  const int split = (((EPI == 1 && !GATHER && !BKN) || (EPI == 2 && BKN)) && part != nullptr &&
                     (B1 == nullptr || !BKN || (K / 2) % BK == 0))
                        ? 2
                        : 1;
  // the 256-row tiles, then at most one 128-row and one 64-row tile per group
  const int64_t main_blocks = cdiv(max_tiles * nb, NXCD) * NXCD;
  const int64_t grid = main_blocks + 2 * static_cast<int64_t>(groups) * nb * split;
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
                     static_cast<int>(main_blocks), B0, B1, group_stride, N, K, C, C2, C3, part,
                     split);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || split == 1) return e;
  hipLaunchKernelGGL(finish_split_kernel<EPI == 2>,
                     dim3(static_cast<unsigned>(groups) * 128u, static_cast<unsigned>(cdiv(N / 8, 256))),
                     dim3(256), 0, st, offsets, groups, N, split, part, C);
  return hipGetLastError();
}

// a_rows: rows of A (of the token matrix when rows are gathered), or -1 if not known
template <int EPI, bool GATHER, bool BKN = false>
hipError_t launch_gemm(const bf16_t* A, const int32_t* gather, const int32_t* offsets,
                       const int32_t* tile_off, int groups, int64_t max_tiles, const bf16_t* B0,
                       const bf16_t* B1, int64_t group_stride, int N, int K, bf16_t* C,
                       hipStream_t st, float* C2 = nullptr, float* C3 = nullptr,
                       int64_t a_rows = -1, float* part = nullptr) {
  if (K % BK == 0)
    return launch_gemm_t<EPI, false, GATHER, BKN>(A, gather, offsets, tile_off, groups, max_tiles,
                                                  B0, B1, group_stride, N, K, C, C2, C3, st,
                                                  a_rows, part);
  return launch_gemm_t<EPI, true, GATHER, BKN>(A, gather, offsets, tile_off, groups, max_tiles, B0,
                                               B1, group_stride, N, K, C, C2, C3, st, a_rows,
                                               part);
}

}  // namespace

hipError_t launch_gemm_up_bf16(int groups, int d, int Mg, const void* rows,
                               const int32_t* gather, const int32_t* offsets,
                               const int32_t* tile_off, int64_t max_tiles, const void* W_gate,
                               const void* W_up, void* h, hipStream_t st, int64_t a_rows) {
  const bf16_t* A = static_cast<const bf16_t*>(rows);
  const bf16_t* Wg = static_cast<const bf16_t*>(W_gate);
  const bf16_t* Wu = static_cast<const bf16_t*>(W_up);
  const int64_t gs = static_cast<int64_t>(Mg) * d;
  bf16_t* H = static_cast<bf16_t*>(h);
  if (gather != nullptr)
    return launch_gemm<0, true>(A, gather, offsets, tile_off, groups, max_tiles, Wg, Wu, gs, Mg, d,
                                H, st, nullptr, nullptr, a_rows);
  return launch_gemm<0, false>(A, nullptr, offsets, tile_off, groups, max_tiles, Wg, Wu, gs, Mg, d,
                               H, st, nullptr, nullptr, a_rows);
}

// G[r] = A_r W_gate[g]^T and U[r] = A_r W_up[g]^T in fp32 (A_r = rows[gather[r]] when gather !=
// NULL): the gate/up tile of the SwiGLU GEMM with the pre-activations stored instead of h (the
// backward's recompute)
hipError_t launch_gemm_gu_f32out_bf16(int groups, int d, int Mg, const void* rows,
                                      const int32_t* gather, const int32_t* offsets,
                                      const int32_t* tile_off, int64_t max_tiles,
                                      const void* W_gate, const void* W_up, float* G, float* U,
                                      hipStream_t st, int64_t a_rows) {
  const bf16_t* A = static_cast<const bf16_t*>(rows);
  const bf16_t* Wg = static_cast<const bf16_t*>(W_gate);
  const bf16_t* Wu = static_cast<const bf16_t*>(W_up);
  const int64_t gs = static_cast<int64_t>(Mg) * d;
  bf16_t* Gp = reinterpret_cast<bf16_t*>(G);  // holds floats (EPI 3)
  if (gather != nullptr)
    return launch_gemm<3, true>(A, gather, offsets, tile_off, groups, max_tiles, Wg, Wu, gs, Mg, d,
                                Gp, st, U, nullptr, a_rows);
  return launch_gemm<3, false>(A, nullptr, offsets, tile_off, groups, max_tiles, Wg, Wu, gs, Mg, d,
                               Gp, st, U, nullptr, a_rows);
}

// The SwiGLU GEMM of launch_gemm_up_bf16 that also stores the fp32 gate and up pre-activations
// G[r] and U[r] (the values launch_gemm_gu_f32out_bf16 computes, from the same accumulators), so
// that a backward can take them instead of recomputing them; h is unchanged.
hipError_t launch_gemm_up_save_bf16(int groups, int d, int Mg, const void* rows,
                                    const int32_t* gather, const int32_t* offsets,
                                    const int32_t* tile_off, int64_t max_tiles, const void* W_gate,
                                    const void* W_up, void* h, float* G, float* U,
                                    hipStream_t st, int64_t a_rows) {
  const bf16_t* A = static_cast<const bf16_t*>(rows);
  const bf16_t* Wg = static_cast<const bf16_t*>(W_gate);
  const bf16_t* Wu = static_cast<const bf16_t*>(W_up);
  const int64_t gs = static_cast<int64_t>(Mg) * d;
  bf16_t* H = static_cast<bf16_t*>(h);
  if (gather != nullptr)
    return launch_gemm<4, true>(A, gather, offsets, tile_off, groups, max_tiles, Wg, Wu, gs, Mg, d,
                                H, st, G, U, a_rows);
  return launch_gemm<4, false>(A, nullptr, offsets, tile_off, groups, max_tiles, Wg, Wu, gs, Mg, d,
                               H, st, G, U, a_rows);
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
                               float* C, hipStream_t st, float* part) {
  const bf16_t* A = static_cast<const bf16_t*>(rows);
  const bf16_t* b0 = static_cast<const bf16_t*>(B0);
  const bf16_t* b1 = static_cast<const bf16_t*>(B1);
  bf16_t* Cp = reinterpret_cast<bf16_t*>(C);  // holds floats (EPI 2)
  // 16-byte column chunks, and a group's row offsets (K rows of N) in 32 bits
  if (N < 8 || N % 8 != 0 || static_cast<int64_t>(K) * N * 2 >= (int64_t{1} << 32))
    return hipErrorInvalidValue;
  if (gather != nullptr)
    return launch_gemm<2, true, true>(A, gather, offsets, tile_off, groups, max_tiles, b0, b1,
                                      group_stride, N, K, Cp, st, nullptr, nullptr, -1, part);
  return launch_gemm<2, false, true>(A, nullptr, offsets, tile_off, groups, max_tiles, b0, b1,
                                     group_stride, N, K, Cp, st, nullptr, nullptr, -1, part);
}

// C_g [Ma][Nb] (fp32) = sum over the rows of group g of A[r][m] B[r][n] (weight gradients): the
// persistent K-major kernel, one block per CU
hipError_t launch_gemm_wgrad_bf16(const void* A, int lda, const void* B, int ldb, int64_t rows,
                                  const int32_t* offsets, const int32_t* kt, int groups, int Ma,
                                  int Nb, float* C, hipStream_t st) {
  constexpr size_t lds = 2 * Geo<256>::STAGE;
  const int64_t pb = persistent_blocks();
  if (pb < NXCD || rows < 1 || rows > INT32_MAX || Ma < 8 || Nb < 8 || Ma % 8 || Nb % 8)
    return hipErrorInvalidValue;
  if (groups <= 0) return hipSuccess;
  static std::atomic<bool> attr{false};
  if (!attr.load(std::memory_order_acquire)) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&wgrad_persistent_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
    attr.store(true, std::memory_order_release);
  }
  const int64_t tiles = static_cast<int64_t>(groups) * cdiv(Ma, 256) * cdiv(Nb, 256);
  const int64_t upper = cdiv(tiles, NXCD) * NXCD;
  const int64_t grid = upper < pb ? upper : pb;
  hipLaunchKernelGGL(wgrad_persistent_kernel, dim3(static_cast<unsigned>(grid)), dim3(NT), lds, st,
                     static_cast<const bf16_t*>(A), lda, static_cast<const bf16_t*>(B), ldb,
                     static_cast<int>(rows), offsets, kt, groups, Ma, Nb, C);
  return hipGetLastError();
}

// part: NULL, or [2][groups][128][d] fp32 for the remainder tiles of a long-K product in K chunks
hipError_t launch_gemm_down_bf16(int groups, int d, int Mg, const int32_t* offsets,
                                 const int32_t* tile_off, int64_t max_tiles, const void* W_down,
                                 const void* h, void* out, hipStream_t st, int64_t a_rows,
                                 float* part) {
  return launch_gemm<1, false>(static_cast<const bf16_t*>(h), nullptr, offsets, tile_off, groups,
                               max_tiles, static_cast<const bf16_t*>(W_down), nullptr,
                               static_cast<int64_t>(Mg) * d, d, Mg, static_cast<bf16_t*>(out), st,
                               nullptr, nullptr, a_rows, part);
}

// The routed gate/up product (rows of x gathered through `gather`) and the shared experts' (all T
// rows of x, one group of width SMg) in one launch, when the persistent kernel serves both;
// otherwise as two launches of launch_gemm_up_bf16.
hipError_t launch_gemm_up_shared_bf16(int groups, int d, int Mg, const void* x,
                                      const int32_t* gather, const int32_t* offsets,
                                      const int32_t* tile_off, int64_t max_tiles,
                                      const void* W_gate, const void* W_up, void* h, int64_t T,
                                      int SMg, const int32_t* sh_offsets,
                                      const int32_t* sh_tile_off, int64_t sh_tiles,
                                      const void* Ws_gate, const void* Ws_up, void* h_sh,
                                      hipStream_t st) {
  const bf16_t* X = static_cast<const bf16_t*>(x);
  GemmProb P0{X, gather, offsets, tile_off, static_cast<const bf16_t*>(W_gate),
              static_cast<const bf16_t*>(W_up), static_cast<int64_t>(Mg) * d,
              static_cast<bf16_t*>(h), groups, Mg, d};
  GemmProb P1{X, nullptr, sh_offsets, sh_tile_off, static_cast<const bf16_t*>(Ws_gate),
              static_cast<const bf16_t*>(Ws_up), static_cast<int64_t>(SMg) * d,
              static_cast<bf16_t*>(h_sh), 1, SMg, d};
  if (gather != nullptr && persistent_ok(P0, T) && persistent_ok(P1, T)) {
    if (d % BK == 0) return launch_persistent<0, false, true>(P0, max_tiles, P1, sh_tiles, st);
    return launch_persistent<0, true, true>(P0, max_tiles, P1, sh_tiles, st);
  }
  hipError_t e = launch_gemm_up_bf16(groups, d, Mg, x, gather, offsets, tile_off, max_tiles, W_gate,
                                     W_up, h, st, T);
  if (e != hipSuccess) return e;
  return launch_gemm_up_bf16(1, d, SMg, x, nullptr, sh_offsets, sh_tile_off, sh_tiles, Ws_gate,
                             Ws_up, h_sh, st, T);
}

// The routed down product (R rows of h) and the shared experts' (T rows of h_sh, K = SMg) in one
// launch when the persistent kernel serves both; otherwise as two launches.
hipError_t launch_gemm_down_shared_bf16(int groups, int d, int Mg, const int32_t* offsets,
                                        const int32_t* tile_off, int64_t max_tiles,
                                        const void* W_down, const void* h, void* out, int64_t R,
                                        int64_t T, int SMg, const int32_t* sh_offsets,
                                        const int32_t* sh_tile_off, int64_t sh_tiles,
                                        const void* Ws_down, const void* h_sh, void* sh,
                                        hipStream_t st, float* part) {
  GemmProb P0{static_cast<const bf16_t*>(h), nullptr, offsets, tile_off,
              static_cast<const bf16_t*>(W_down), nullptr, static_cast<int64_t>(Mg) * d,
              static_cast<bf16_t*>(out), groups, d, Mg};
  GemmProb P1{static_cast<const bf16_t*>(h_sh), nullptr, sh_offsets, sh_tile_off,
              static_cast<const bf16_t*>(Ws_down), nullptr, static_cast<int64_t>(SMg) * d,
              static_cast<bf16_t*>(sh), 1, d, SMg};
  if (persistent_ok(P0, R) && persistent_ok(P1, T)) {
    if (Mg % BK == 0 && SMg % BK == 0)
      return launch_persistent<1, false, false>(P0, max_tiles, P1, sh_tiles, st);
    return launch_persistent<1, true, false>(P0, max_tiles, P1, sh_tiles, st);
  }
  hipError_t e = launch_gemm_down_bf16(groups, d, Mg, offsets, tile_off, max_tiles, W_down, h, out,
                                       st, R, part);
  if (e != hipSuccess) return e;
  return launch_gemm_down_bf16(1, d, SMg, sh_offsets, sh_tile_off, sh_tiles, Ws_down, h_sh, sh, st,
                               T, nullptr);
}

}  // namespace moe

// Router kernel: l = x W_r^T, max-subtracted softmax with log-sum-exp, biased top-k selection,
// renormalised gates and per-block partial statistics ("MoE：条件计算与路由" §原理与演进,
// §无辅助损失负载均衡（ALF-LB）, §7 eqs. (1)-(2); "MOE大模型对比篇" §2.2 for the LSE term).
// With sigmoid scoring (the DeepSeek-V3 gate of the adg.csdn.net notes page, §九) each expert's
// score is 1 / (1 + exp(-l)) on its own; selection, bias and renormalisation are unchanged, the
// probability statistic uses the scores normalised over the experts, and lse still feeds z.
//
// A block owns TB consecutive tokens (bf16: 8 waves, 16 tokens when E <= 16, else 64; fp32: 4
// waves, 64 tokens). The logits tile [TB x E] never leaves the chip: bf16 inputs go through
// v_mfma_f32_16x16x32_bf16 with the hidden dimension split across the waves; fp32 inputs use
// plain FMA loops. Then every thread of the block works on the routing: a group of lanes shares a
// token, each lane walking a strided share of the experts, and butterflies combine the group's
// maximum, exp-sum and top-k (equal scores go to the lower expert index). Statistics leave as
// per-block partials (expert histogram, sum of g, sum of lse^2) reduced later in a fixed order, so
// every result is bit-reproducible.
#include "moe_internal.h"

#include <math.h>

#include <type_traits>

namespace moe {
namespace {

constexpr int RT = kRouteTokens;  // 64 tokens per fp32 block

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Calls f(std::integral_constant<int, I>) for I = B .. E-1 (register rings need constant slots).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// XOR butterflies over aligned groups of G lanes: every lane of a group ends with the same bits
// (each step combines the same two values, in either order, with a commutative operation).
template <int G>
__device__ __forceinline__ float bfly_max(float v) {
#pragma unroll
  for (int s = 1; s < G; s <<= 1) v = fmaxf(v, __shfl_xor(v, s));
  return v;
}
template <int G>
__device__ __forceinline__ float bfly_sum(float v) {
#pragma unroll
  for (int s = 1; s < G; s <<= 1) v += __shfl_xor(v, s);
  return v;
}

// ------------------------------------------------------------------------------------------
// Per-token routing over the logits tile in LDS, shared by every router kernel. G consecutive
// lanes share a token (G = threads / TB, a power of two up to 64, so a token's lanes sit in one
// wave) and lane j of the group owns experts j, j + G, j + 2G, ... . The maximum m and the sum of
// exp(l - m) over the experts (lse = m + ln sum) are formed per lane in index order and combined by
// butterflies. Each lane then writes its scores g_e = exp(l_e - lse) (sigmoid scoring:
// 1 / (1 + exp(-l_e))) back over the logits and keeps its best KM selection scores s_e = g_e + b_e,
// sorted. The top-k is k rounds of a butterfly arg-max under one total order, higher s first and
// equal s to the lower expert index (the order a walk over the experts in index order with a
// strict comparison selects in): each lane offers its best expert not yet taken and the winner's
// owner drops it, so slot j holds the j-th expert of that order. Block partials: the expert
// histogram (LDS integer atomics: order-free), per expert the sum over the block's tokens of g_e
// (sigmoid: g_e / sum_e' g_e'), and the sums of lse^2 and of the routing entropy, each reduced in
// a fixed tree, so every result is bit-reproducible.
//   L: [TB][Ls] fp32 logits; hcnt: >= E ints; lsq, hsq: TB floats.
//   flags: kRouteRenorm | kRouteSigmoid | kRouteExpertChoice (score columns instead of top-k).
// ------------------------------------------------------------------------------------------
template <int KM, int G>
__device__ void route_tokens(float* L, int Ls, int TB, int64_t t0, int64_t T, int E, int k,
                             int flags, const float* __restrict__ b,
                             int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
                             int32_t* __restrict__ hist, float* __restrict__ gpart,
                             float* __restrict__ lpart, float* __restrict__ hpart,
                             float* __restrict__ cols, int* hcnt, float* lsq, float* hsq) {
  static_assert(G >= 1 && G <= 64 && (G & (G - 1)) == 0, "lanes per token");
  const int tid = threadIdx.x;
  const int tl = tid / G, j = tid % G;  // blockDim.x == TB G
  const int64_t t = t0 + tl;
  const bool live = t < T;
  const bool sig = (flags & kRouteSigmoid) != 0;
  const bool ec = (flags & kRouteExpertChoice) != 0;
  for (int e = tid; e < E; e += blockDim.x) hcnt[e] = 0;
  __syncthreads();
  float* row = L + tl * Ls;
  float m = -INFINITY;
  for (int e = j; e < E; e += G) m = fmaxf(m, row[e]);
  m = bfly_max<G>(m);
  float sum = 0.f;
  for (int e = j; e < E; e += G) sum += expf(row[e] - m);
  sum = bfly_sum<G>(sum);
  const float lse = m + logf(sum);
  float cv[KM], cg[KM];  // this lane's best selection scores and their g, best first
  int ci[KM];
#pragma unroll
  for (int q = 0; q < KM; ++q) {
    cv[q] = -INFINITY;
    cg[q] = 0.f;
    ci[q] = 0x7fffffff;
  }
  float ssum = 0.f;  // sigmoid: sum of the scores over the experts
  float hacc = 0.f;  // entropy term: softmax sum g (l - lse); sigmoid sum s ln s
  for (int e = j; e < E; e += G) {
    const float l = row[e];
    const float g = sig ? 1.f / (1.f + expf(-l)) : expf(l - lse);
    row[e] = g;
    if (sig) ssum += g;
    hacc += sig ? (g > 0.f ? g * logf(g) : 0.f) : g * (l - lse);
    if (ec) {  // expert choice: columns of logits and scores for the per-expert selection
      if (live) {
        cols[static_cast<int64_t>(e) * T + t] = l;
        cols[(static_cast<int64_t>(E) + e) * T + t] = g;
      }
    } else {
      // sorted insertion; this lane's experts arrive in ascending index order, so a strict
      // comparison keeps equal scores in index order
      const float v = b != nullptr ? g + b[e] : g;
      static_for<1, KM>([&](auto qc) __attribute__((always_inline)) {
        constexpr int q = KM - decltype(qc)::value;  // KM - 1 down to 1
        const bool up = v > cv[q - 1], here = v > cv[q];
        cv[q] = up ? cv[q - 1] : (here ? v : cv[q]);
        cg[q] = up ? cg[q - 1] : (here ? g : cg[q]);
        ci[q] = up ? ci[q - 1] : (here ? e : ci[q]);
      });
      const bool top = v > cv[0];
      cv[0] = top ? v : cv[0];
      cg[0] = top ? g : cg[0];
      ci[0] = top ? e : ci[0];
    }
  }
  ssum = bfly_sum<G>(ssum);
  hacc = bfly_sum<G>(hacc);
  if (!ec) {
    int we[KM];
    float wg[KM];
    float wsum = 0.f;
    static_for<0, KM>([&](auto rc) __attribute__((always_inline)) {
      constexpr int r = decltype(rc)::value;
      we[r] = 0;
      wg[r] = 0.f;
      if (r < k) {
        float v = cv[0], g = cg[0];
        int e = ci[0];
#pragma unroll
        for (int sh = 1; sh < G; sh <<= 1) {
          const float v2 = __shfl_xor(v, sh), g2 = __shfl_xor(g, sh);
          const int e2 = __shfl_xor(e, sh);
          const bool take = v2 > v || (v2 == v && e2 < e);
          v = take ? v2 : v;
          g = take ? g2 : g;
          e = take ? e2 : e;
        }
        we[r] = e;
        wg[r] = g;
        wsum += g;  // slot order
        const bool mine = ci[0] == e;  // expert e has one owner
        // the shift is spelled with constant indices throughout: a select between neighbouring
        // elements under a loop index is otherwise folded into a variable index, which sends the
        // whole list to scratch memory
        static_for<0, KM - 1>([&](auto qc) __attribute__((always_inline)) {
          constexpr int q = decltype(qc)::value;
          cv[q] = mine ? cv[q + 1] : cv[q];
          cg[q] = mine ? cg[q + 1] : cg[q];
          ci[q] = mine ? ci[q + 1] : ci[q];
        });
        cv[KM - 1] = mine ? -INFINITY : cv[KM - 1];
        ci[KM - 1] = mine ? 0x7fffffff : ci[KM - 1];
      }
    });
    const bool renorm = (flags & kRouteRenorm) != 0;
    static_for<0, KM>([&](auto rc) __attribute__((always_inline)) {
      constexpr int r = decltype(rc)::value;
      if (r < k && r % G == j && live) {
        topk_idx[t * k + r] = we[r];
        topk_w[t * k + r] = renorm ? wg[r] / wsum : wg[r];
        atomicAdd(&hcnt[we[r]], 1);
      }
    });
  }
  if (sig) {  // the probability statistic uses the scores normalised over the experts
    const float inv = 1.f / ssum;
    for (int e = j; e < E; e += G) row[e] *= inv;
  }
  if (j == 0) {
    lsq[tl] = live ? lse * lse : 0.f;
    // routing entropy of the token's distribution (softmax g, or s / sum s)
    hsq[tl] = live ? (sig ? logf(ssum) - hacc / ssum : -hacc) : 0.f;
  }
  __syncthreads();
  // per-expert sums over the block's tokens: 8 lanes per expert each sum a run of tokens in order,
  // then a butterfly
  const int64_t blk = blockIdx.x;
  const int nt = static_cast<int>(min<int64_t>(TB, T - t0));
  constexpr int PE = 8;
  const int per = (TB + PE - 1) / PE;
  const int ep = tid / PE, pp = tid % PE;
  for (int base = 0; base < E; base += static_cast<int>(blockDim.x) / PE) {
    const int e = base + ep;
    float gs = 0.f;
    if (e < E) {
      for (int q = 0; q < per; ++q) {
        const int tq = pp * per + q;
        if (tq < nt) gs += L[tq * Ls + e];
      }
    }
    gs = bfly_sum<PE>(gs);
    if (pp == 0 && e < E) {
      gpart[blk * E + e] = gs;
      hist[blk * E + e] = hcnt[e];
    }
  }
  if (tid < 64) {  // TB <= 64
    const float ls = bfly_sum<64>(tid < nt ? lsq[tid] : 0.f);
    const float hs = bfly_sum<64>(tid < nt ? hsq[tid] : 0.f);
    if (tid == 0) {
      lpart[blk] = ls;
      hpart[blk] = hs;
    }
  }
}

// The top-k list length of a kernel (KM = 2, 8 or 16 slots, k <= KM) is a template argument
// chosen on the host: one per-token routine per kernel keeps each kernel small (three inlined
// copies in one kernel take the device compiler tens of minutes).
template <typename F>
hipError_t with_km(int k, F&& f) {
  if (k <= 2) return f(std::integral_constant<int, 2>{});
  if (k <= 8) return f(std::integral_constant<int, 8>{});
  return f(std::integral_constant<int, 16>{});
}

// logits row stride: 8 banks apart, so the 8 lanes of each of a wave's 8 tokens (lane j reading
// expert j + 8 i of its token's row) hit 64 distinct banks
constexpr int kLogitsStride = MOE_E_MAX + 8;

// ------------------------------------------------------------------------------------------
// bf16: logits on MFMA. A block owns TB = 16 MB tokens; its eight waves split the hidden dimension
// into eight contiguous ranges of 32-wide k-steps and load their MFMA operands straight from
// global memory (x rows of the block's tokens, W_r rows of every expert), so no barrier sits in
// the k loop. The eight partial logit tiles are summed in LDS in wave order (fixed, so results are
// reproducible). Fragment layout of v_mfma_f32_16x16x32_bf16: lane l supplies row (l % 16) of A
// and column (l % 16) of B with 8 consecutive k of k-group (l / 16); result element
// (row 4*(l/16) + j, column l % 16) lands in lane l, register j.
// ------------------------------------------------------------------------------------------
constexpr int kRouteThreads = 512;  // 8 waves: K is split 8 ways, two waves per SIMD

template <int MB, int NEB, int NG, int KM>
__global__ __launch_bounds__(kRouteThreads) void route_bf16_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ W, const float* __restrict__ b,
    int64_t T, int d, int E, int k, int flags, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, int32_t* __restrict__ hist, float* __restrict__ gpart,
    float* __restrict__ lpart, float* __restrict__ hpart, float* __restrict__ cols) {
  constexpr int TB = 16 * MB;
  constexpr int NW = kRouteThreads / 64;
  constexpr int NWK = NW / NG;                // waves splitting K within an expert group
  constexpr int NEBG = (NEB + NG - 1) / NG;   // expert blocks of 16 per group
  __shared__ float L[TB * kLogitsStride];
  __shared__ int hcnt[MOE_E_MAX];
  __shared__ float lsq[TB];
  __shared__ float hsq[TB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = wave / NWK, kw = wave % NWK;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * TB;
  const int r16 = lane & 15, kg = lane >> 4;

  const bf16_t* xr[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    int64_t t = t0 + m * 16 + r16;
    t = t < T ? t : T - 1;
    xr[m] = x + t * d + kg * 8;
  }
  const bf16_t* wr[NEBG];
  bool wv[NEBG];
#pragma unroll
  for (int j = 0; j < NEBG; ++j) {
    const int e = (grp * NEBG + j) * 16 + r16;
    wv[j] = e < E;
    wr[j] = W + static_cast<int64_t>(wv[j] ? e : 0) * d + kg * 8;
  }
  f32x4 acc[MB][NEBG];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int j = 0; j < NEBG; ++j) acc[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nks = (d + 31) / 32;
  const int s0 = kw * nks / NWK, s1 = (kw + 1) * nks / NWK;
  const bf16x8 zero = {};
  auto load = [&](int s, bf16x8* a, bf16x8* bb) __attribute__((always_inline)) {
    const int kk = s * 32;
    const bool in = kk + kg * 8 < d;  // d is a multiple of 8: a lane's 8 values are all in or out
#pragma unroll
    for (int m = 0; m < MB; ++m) a[m] = in ? *reinterpret_cast<const bf16x8*>(xr[m] + kk) : zero;
#pragma unroll
    for (int j = 0; j < NEBG; ++j)
      bb[j] = (in && wv[j]) ? *reinterpret_cast<const bf16x8*>(wr[j] + kk) : zero;
  };
  auto mma = [&](const bf16x8* a, const bf16x8* bb) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int j = 0; j < NEBG; ++j)
        acc[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[m], bb[j], acc[m][j], 0, 0, 0);
  };
  // a ring of PF k-steps of operands in registers: the loads run PF steps ahead of the MFMAs, so a
  // wave's whole K range (16 steps at d = 4096) is in flight at once
  constexpr int PF = 16;
  bf16x8 ra[PF][MB], rb[PF][NEBG];
  static_for<0, PF>([&](auto pc) __attribute__((always_inline)) {
    constexpr int P = decltype(pc)::value;
    if (s0 + P < s1) load(s0 + P, ra[P], rb[P]);
  });
  for (int base = s0; base < s1; base += PF) {
    static_for<0, PF>([&](auto jc) __attribute__((always_inline)) {
      constexpr int J = decltype(jc)::value;
      const int s = base + J;
      if (s < s1) {
        mma(ra[J], rb[J]);
        if (s + PF < s1) load(s + PF, ra[J], rb[J]);
      }
    });
  }

  // sum the partial tiles of each expert group in wave (K) order; groups own disjoint columns.
  // Every wave parks its tile in LDS, then each element is summed over the K waves in order.
  __shared__ float part[NW * TB * 16 * NEBG];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int j = 0; j < NEBG; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        part[((wave * MB + m) * NEBG + j) * 256 + (kg * 4 + r) * 16 + r16] = acc[m][j][r];
  __syncthreads();
  for (int i = tid; i < NG * MB * NEBG * 256; i += kRouteThreads) {
    const int g = i / (MB * NEBG * 256), rem = i % (MB * NEBG * 256);
    const int m = rem / (NEBG * 256), j = (rem / 256) % NEBG, e16 = rem % 256;
    const int row = e16 / 16, c16 = e16 % 16;
    if (g * NEBG + j < NEB) {
      float v = 0.f;
      for (int q = 0; q < NWK; ++q) {
        const int w = g * NWK + q;
        v = (q == 0) ? part[((w * MB + m) * NEBG + j) * 256 + row * 16 + c16]
                     : v + part[((w * MB + m) * NEBG + j) * 256 + row * 16 + c16];
      }
      L[(m * 16 + row) * kLogitsStride + (g * NEBG + j) * 16 + c16] = v;
    }
  }
  __syncthreads();
  route_tokens<KM, kRouteThreads / TB>(L, kLogitsStride, TB, t0, T, E, k, flags, b, topk_idx,
                                       topk_w, hist, gpart, lpart, hpart, cols, hcnt, lsq, hsq);
}

// ------------------------------------------------------------------------------------------
// fp32: logits by sequential FMA over the hidden dimension (one (token, expert) pair per thread).
// ------------------------------------------------------------------------------------------
template <int KM>
__global__ __launch_bounds__(256) void route_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ W, const float* __restrict__ b,
    int64_t T, int d, int E, int k, int flags, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, int32_t* __restrict__ hist, float* __restrict__ gpart,
    float* __restrict__ lpart, float* __restrict__ hpart, float* __restrict__ cols) {
  __shared__ float L[RT * kLogitsStride];
  __shared__ int hcnt[MOE_E_MAX];
  __shared__ float lsq[RT];
  __shared__ float hsq[RT];
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * RT;  // fp32 blocks are 64 tokens
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
  route_tokens<KM, 256 / RT>(L, kLogitsStride, RT, t0, T, E, k, flags, b, topk_idx, topk_w, hist,
                             gpart, lpart, hpart, cols, hcnt, lsq, hsq);
}

// ------------------------------------------------------------------------------------------
// bf16 with many experts (E > 16): W_r is shared through LDS. A block owns TB tokens (64, or 32
// when E <= 64 and 64-token blocks would leave CUs idle); its eight waves are TB / 16 token blocks
// of 16 times 8 / (TB / 16) expert groups, and each runs the whole hidden dimension, so x is
// streamed once and W_r once per block. The x and W_r k-slices (128 wide where two
// stages fit in 120 KB, else 64: longer contiguous row reads) pass through two LDS stages (rows
// padded by 8 bf16: the 16x16x32 fragment reads are bank-conflict-free) with the next slices
// prefetched into a register ring two deep; one barrier per k-step.
// ------------------------------------------------------------------------------------------
// k per step: 128 where two stages of (TB + 16 NEB) padded rows fit in 120 KB, else 64; and the
// depth of the register ring of k-slices in flight
constexpr int kRouteSliceK = 128, kRouteRing = 2;
template <int NEB, int TB>
constexpr int route_sk() {
  return 2 * (TB + 16 * NEB) * (kRouteSliceK + 8) * 2 <= 120 * 1024 ? kRouteSliceK : 64;
}

template <int NEB, int KM, int TB>
__global__ __launch_bounds__(kRouteThreads) void route_bf16_lds_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ W, const float* __restrict__ b,
    int64_t T, int d, int E, int k, int flags, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, int32_t* __restrict__ hist, float* __restrict__ gpart,
    float* __restrict__ lpart, float* __restrict__ hpart, float* __restrict__ cols) {
  static_assert(TB == 32 || TB == 64, "token blocks of the many-expert router");
  constexpr int kSK = route_sk<NEB, TB>();  // k per step
  constexpr int kSKP = kSK + 8;         // padded LDS row (bf16 elements)
  constexpr int ROWS = TB + 16 * NEB;                 // x rows then W_r rows of a stage
  constexpr int STAGE = ROWS * kSKP;                  // bf16 elements
  constexpr int CPR = kSK / 8;                        // 16-byte chunks per row of a stage
  constexpr int CH = ROWS * CPR;                      // 16-byte chunks per stage
  constexpr int CPT = (CH + kRouteThreads - 1) / kRouteThreads;
  constexpr int TBLK = TB / 16;                       // 16-token blocks: 4 or 2
  constexpr int EG = 8 / TBLK;                        // expert groups over the waves: 2 or 4
  constexpr int NEBH = (NEB + EG - 1) / EG;           // expert blocks per wave
  constexpr int kStagesBytes = 2 * STAGE * 2;
  constexpr int kLBytes = TB * kLogitsStride * 4;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kStagesBytes > kLBytes ? kStagesBytes : kLBytes];
  __shared__ int hcnt[MOE_E_MAX];
  __shared__ float lsq[TB];
  __shared__ float hsq[TB];
  bf16_t* st = reinterpret_cast<bf16_t*>(smem);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tb = wave % TBLK, eh = wave / TBLK;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * TB;
  const int r16 = lane & 15, kg = lane >> 4;

  // chunk c of a stage: row c / CPR (x rows 0..63, then W_r rows), 8 bf16 at column (c % CPR) * 8
  const bf16_t* src[CPT];
  bool ok[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = i * kRouteThreads + tid, r = c / CPR, col = (c % CPR) * 8;
    ok[i] = c < CH;
    if (r < TB) {
      int64_t t = t0 + r;
      t = t < T ? t : T - 1;
      src[i] = x + t * d + col;
    } else {
      const int e = r - TB;
      ok[i] = ok[i] && e < E;
      src[i] = W + static_cast<int64_t>(e < E ? e : 0) * d + col;
    }
  }
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  // a ring of PF k-slices in registers ahead of the two LDS stages: a k-step's MFMA work is short
  // next to the memory latency, so several slices must be in flight
  constexpr int PF = kRouteRing;
  u32x4 rg[PF][CPT];
  auto gload = [&](u32x4 (&r)[CPT], int k0) __attribute__((always_inline)) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int col = ((i * kRouteThreads + tid) % CPR) * 8;
      r[i] = (ok[i] && k0 + col < d) ? *reinterpret_cast<const u32x4*>(src[i] + k0) : zero;
    }
  };
  auto lstore = [&](const u32x4 (&r)[CPT], int stage) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = i * kRouteThreads + tid;
      if (c < CH) *reinterpret_cast<u32x4*>(st + stage * STAGE + (c / CPR) * kSKP + (c % CPR) * 8) = r[i];
    }
  };
  f32x4 acc[NEBH];
#pragma unroll
  for (int j = 0; j < NEBH; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int stage) __attribute__((always_inline)) {
    const bf16_t* sx = st + stage * STAGE + (tb * 16 + r16) * kSKP;
    const bf16_t* sw = st + stage * STAGE + (TB + r16) * kSKP;
#pragma unroll
    for (int sub = 0; sub < kSK / 32; ++sub) {
      const int kc = sub * 32 + kg * 8;
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(sx + kc);
#pragma unroll
      for (int j = 0; j < NEBH; ++j) {
        const int eb = eh * NEBH + j;
        if (eb < NEB) {
          const bf16x8 bb = *reinterpret_cast<const bf16x8*>(sw + eb * 16 * kSKP + kc);
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bb, acc[j], 0, 0, 0);
        }
      }
    }
  };
  const int nk = (d + kSK - 1) / kSK;
  // k-slice j sits in ring slot j % PF from its load until its LDS store one k-step before use
  static_for<0, PF>([&](auto pc) __attribute__((always_inline)) {
    constexpr int P = decltype(pc)::value;
    if (P < nk) gload(rg[P], P * kSK);
  });
  lstore(rg[0], 0);
  if (PF < nk) gload(rg[0], PF * kSK);
  __syncthreads();
  for (int base = 0; base < nk; base += PF) {
    static_for<0, PF>([&](auto jc) __attribute__((always_inline)) {
      constexpr int J = decltype(jc)::value;
      constexpr int NEXT = (J + 1) % PF;  // ring slot of k-slice ks + 1
      const int ks = base + J;
      if (ks < nk) {
        if (ks + 1 < nk) {
          lstore(rg[NEXT], (ks + 1) & 1);  // stage read by k-step ks - 1, behind the barrier
          if (ks + 1 + PF < nk) gload(rg[NEXT], (ks + 1 + PF) * kSK);
        }
        compute(ks & 1);
        __syncthreads();
      }
    });
  }
  float* L = reinterpret_cast<float*>(smem);  // reuses the stages
#pragma unroll
  for (int j = 0; j < NEBH; ++j) {
    const int eb = eh * NEBH + j;
    if (eb < NEB) {
#pragma unroll
      for (int r = 0; r < 4; ++r) L[(tb * 16 + kg * 4 + r) * kLogitsStride + eb * 16 + r16] = acc[j][r];
    }
  }
  __syncthreads();
  route_tokens<KM, kRouteThreads / TB>(L, kLogitsStride, TB, t0, T, E, k, flags, b, topk_idx,
                                       topk_w, hist, gpart, lpart, hpart, cols, hcnt, lsq, hsq);
}

template <int NEB>
hipError_t launch_bf16_lds(hipStream_t st, const void* x, const void* W, const float* b, int64_t T,
                           int d, int E, int k, int flags, int32_t* topk_idx, float* topk_w,
                           int32_t* hist, float* gpart, float* lpart, float* hpart,
                           float* cols) {
  const int tbt = route_block_tokens(MOE_BF16, E, T);
  const dim3 grid(static_cast<unsigned>(cdiv(T, tbt)));
  return with_km(k, [&](auto km) {
    if (tbt == 32)
      hipLaunchKernelGGL((route_bf16_lds_kernel<NEB, decltype(km)::value, 32>), grid,
                         dim3(kRouteThreads), 0, st, static_cast<const bf16_t*>(x),
                         static_cast<const bf16_t*>(W), b, T, d, E, k, flags, topk_idx, topk_w,
                         hist, gpart, lpart, hpart, cols);
    else
      hipLaunchKernelGGL((route_bf16_lds_kernel<NEB, decltype(km)::value, 64>), grid,
                         dim3(kRouteThreads), 0, st, static_cast<const bf16_t*>(x),
                         static_cast<const bf16_t*>(W), b, T, d, E, k, flags, topk_idx, topk_w,
                         hist, gpart, lpart, hpart, cols);
    return hipGetLastError();
  });
}

template <int MB, int NEB, int NG>
hipError_t launch_bf16(hipStream_t st, const void* x, const void* W, const float* b,
                       int64_t T, int d, int E, int k, int flags, int32_t* topk_idx,
                       float* topk_w, int32_t* hist, float* gpart, float* lpart, float* hpart,
                           float* cols) {
  const int64_t nblk = cdiv(T, 16 * MB);
  return with_km(k, [&](auto km) {
    hipLaunchKernelGGL((route_bf16_kernel<MB, NEB, NG, decltype(km)::value>),
                       dim3(static_cast<unsigned>(nblk)), dim3(kRouteThreads), 0, st,
                       static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(W), b, T, d, E,
                       k, flags, topk_idx, topk_w, hist, gpart, lpart, hpart, cols);
    return hipGetLastError();
  });
}

}  // namespace

// Tokens per router block: fp32 64; bf16 16 for E <= 16, else 64, or 32 when 64-token blocks would
// leave CUs idle (fewer than 512 blocks, two per CU) and W_r is small (E <= 64: every block streams
// all of it, so halving the blocks' tokens doubles that traffic; with 160 or 256 experts that cost
// more than the idle CUs did)
int route_block_tokens(int dtype, int E, int64_t T) {
  if (dtype == MOE_F32) return RT;
  if (E <= 16) return 16;
  return (E <= 64 && cdiv(T, 64) < 512) ? 32 : 64;
}

hipError_t launch_route(int dtype, int64_t T, int d, int E, int k, int flags, const void* x,
                        const void* W_r, const float* b, int32_t* topk_idx, float* topk_w,
                        int32_t* hist, float* gpart, float* lpart, float* hpart,
                        float* cols, hipStream_t st) {
  if (dtype == MOE_F32) {
    const int64_t nblk = cdiv(T, RT);
    return with_km(k, [&](auto km) {
      hipLaunchKernelGGL((route_f32_kernel<decltype(km)::value>), dim3(static_cast<unsigned>(nblk)),
                         dim3(256), 0, st, static_cast<const float*>(x),
                         static_cast<const float*>(W_r), b, T, d, E, k, flags, topk_idx, topk_w,
                         hist, gpart, lpart, hpart, cols);
      return hipGetLastError();
    });
  }
  const int neb = static_cast<int>(cdiv(E, 16));
#define MOE_ROUTE_CASE(N)                                                                   \
  case N:                                                                                   \
    return launch_bf16_lds<N>(st, x, W_r, b, T, d, E, k, flags, topk_idx, topk_w, hist, gpart, \
                              lpart, hpart, cols);
  // up to 16 experts: 16-token blocks with the hidden dimension split over the waves (more blocks
  // in flight); more: 64-token blocks with W_r shared through LDS
  if (E <= 16)
    return launch_bf16<1, 1, 1>(st, x, W_r, b, T, d, E, k, flags, topk_idx, topk_w, hist, gpart,
                                lpart, hpart, cols);
  switch (neb) {
    MOE_ROUTE_CASE(2) MOE_ROUTE_CASE(3) MOE_ROUTE_CASE(4) MOE_ROUTE_CASE(5) MOE_ROUTE_CASE(6)
    MOE_ROUTE_CASE(7) MOE_ROUTE_CASE(8) MOE_ROUTE_CASE(9) MOE_ROUTE_CASE(10) MOE_ROUTE_CASE(11)
    MOE_ROUTE_CASE(12) MOE_ROUTE_CASE(13) MOE_ROUTE_CASE(14) MOE_ROUTE_CASE(15) MOE_ROUTE_CASE(16)
    default: return hipErrorInvalidValue;
  }
#undef MOE_ROUTE_CASE
}

}  // namespace moe

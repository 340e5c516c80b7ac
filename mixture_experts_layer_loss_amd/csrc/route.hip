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
// plain FMA loops. Then one lane per token walks the experts in index order (softmax maximum and
// sum, then a sorted top-k insertion in registers), so equal scores go to the lower expert index
// and no cross-lane operation sits on the per-token path. Statistics leave as per-block partials
// (expert histogram, sum of g, sum of lse^2) reduced later in a fixed order, so every result is
// bit-reproducible.
#include "moe_internal.h"

#include <math.h>

#include <type_traits>

namespace moe {
namespace {

constexpr int RT = kRouteTokens;  // 64 tokens per fp32 block

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Insert score v of expert e into a list of KM scores sorted in descending order. Experts arrive
// in ascending index order and only a strictly larger score moves an entry down, so equal scores
// stay ordered by index (ties go to the lower expert index). Branch-free; NaN never enters.
template <int KM>
__device__ __forceinline__ void topk_insert(float v, int e, float (&tv)[KM], int (&ti)[KM]) {
#pragma unroll
  for (int j = KM - 1; j >= 1; --j) {
    const bool beats_prev = v > tv[j - 1];  // entry j-1 moves down to j
    const bool beats = v > tv[j];
    tv[j] = beats_prev ? tv[j - 1] : (beats ? v : tv[j]);
    ti[j] = beats_prev ? ti[j - 1] : (beats ? e : ti[j]);
  }
  const bool top = v > tv[0];
  tv[0] = top ? v : tv[0];
  ti[0] = top ? e : ti[0];
}

// Calls f(std::integral_constant<int, I>) for I = B .. E-1 (register rings need constant slots).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// ------------------------------------------------------------------------------------------
// Per-token routing over the logits tile in LDS, shared by both dtypes. One lane per token:
// wave w takes tokens [w TB/4, (w+1) TB/4) of the block's TB. The lane walks the experts in index
// order: maximum, sum of exp(l - m) (so lse = m + ln sum), then g_e = exp(l_e - lse) or, with
// sigmoid scoring, g_e = 1 / (1 + exp(-l_e)) (written back over the logit), s_e = g_e + b_e and the
// sorted top-KM insertion; k <= KM. Block partials: the expert histogram (LDS integer atomics:
// order-free), sum over tokens of g_e (sigmoid: g_e / sum_e' g_e') per expert and sum of lse^2,
// the latter two summed in token order.
//   L: [TB][Ls] fp32; scratch: >= MOE_E_MAX ints + 64 floats. flags: kRouteRenorm | kRouteSigmoid.
// ------------------------------------------------------------------------------------------
template <int KM>
__device__ void route_tokens(float* L, int Ls, int TB, int64_t t0, int64_t T, int E, int k,
                             int flags, const float* __restrict__ b,
                             int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
                             int32_t* __restrict__ hist, float* __restrict__ gpart,
                             float* __restrict__ lpart, float* __restrict__ hpart,
                             float* __restrict__ cols, int* hcnt, float* lsq, float* hsq) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int tpw = TB / nw;
  for (int e = threadIdx.x; e < E; e += blockDim.x) hcnt[e] = 0;
  __syncthreads();
  if (lane < tpw) {
    const int tl = wave * tpw + lane;
    const int64_t t = t0 + tl;
    float lse2 = 0.f, ent = 0.f;
    if (t < T) {
      float* row = L + tl * Ls;  // Ls % 4 == 0: 16-byte aligned; the pad past E holds -inf
      const int E4 = (E + 3) & ~3;
      float m = -INFINITY;
#pragma unroll 4
      for (int e = 0; e < E4; e += 4) {
        const float4 v = *reinterpret_cast<const float4*>(row + e);
        m = fmaxf(m, fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)));
      }
      float sum = 0.f;
#pragma unroll 4
      for (int e = 0; e < E4; e += 4) {
        const float4 v = *reinterpret_cast<const float4*>(row + e);
        sum += expf(v.x - m);
        sum += expf(v.y - m);
        sum += expf(v.z - m);
        sum += expf(v.w - m);
      }
      const float lse = m + logf(sum);
      lse2 = lse * lse;
      float tv[KM];
      int ti[KM];
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        tv[j] = -INFINITY;
        ti[j] = 0;
      }
      const bool sig = (flags & kRouteSigmoid) != 0;
      const bool ec = (flags & kRouteExpertChoice) != 0;
      float ssum = 0.f;  // sigmoid: sum of the scores over the experts (the pad adds 0)
      float hacc = 0.f;  // entropy term: softmax sum g (l - lse); sigmoid sum s ln s
      for (int e = 0; e < E4; e += 4) {
        float4 v = *reinterpret_cast<const float4*>(row + e);
        const float l4[4] = {v.x, v.y, v.z, v.w};
        if (sig) {
          v.x = 1.f / (1.f + expf(-v.x));
          v.y = 1.f / (1.f + expf(-v.y));
          v.z = 1.f / (1.f + expf(-v.z));
          v.w = 1.f / (1.f + expf(-v.w));
          ssum += v.x;
          ssum += v.y;
          ssum += v.z;
          ssum += v.w;
        } else {
          v.x = expf(v.x - lse);
          v.y = expf(v.y - lse);
          v.z = expf(v.z - lse);
          v.w = expf(v.w - lse);
        }
        *reinterpret_cast<float4*>(row + e) = v;
        const float g4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ee = e + q;
          if (ee < E) {
            if (ec) {  // expert choice: columns of logits and scores for the per-expert selection
              cols[static_cast<int64_t>(ee) * T + t] = l4[q];
              cols[(static_cast<int64_t>(E) + ee) * T + t] = g4[q];
            } else {
              topk_insert<KM>(b != nullptr ? g4[q] + b[ee] : g4[q], ee, tv, ti);
            }
            hacc += sig ? (g4[q] > 0.f ? g4[q] * logf(g4[q]) : 0.f) : g4[q] * (l4[q] - lse);
          }
        }
      }
      // routing entropy of the token's distribution (softmax g, or s / sum s)
      ent = sig ? logf(ssum) - hacc / ssum : -hacc;
      float wsum = 0.f;
#pragma unroll
      for (int j = 0; j < KM; ++j)
        if (j < k) wsum += row[ti[j]];
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        if (j < k && !ec) {
          const float gj = row[ti[j]];
          topk_idx[t * k + j] = ti[j];
          topk_w[t * k + j] = (flags & kRouteRenorm) ? gj / wsum : gj;
          atomicAdd(&hcnt[ti[j]], 1);
        }
      }
      if (sig) {  // the probability statistic uses the scores normalised over the experts
        const float inv = 1.f / ssum;
        for (int e = 0; e < E4; ++e) row[e] *= inv;
      }
    }
    lsq[tl] = lse2;
    hsq[tl] = ent;
  }
  __syncthreads();
  const int64_t blk = blockIdx.x;
  const int nt = static_cast<int>(min<int64_t>(TB, T - t0));
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    float gs = 0.f;
    for (int tl = 0; tl < nt; ++tl) gs += L[tl * Ls + e];
    gpart[blk * E + e] = gs;
    hist[blk * E + e] = hcnt[e];
  }
  if (threadIdx.x == 0) {
    float ls = 0.f, hs = 0.f;
    for (int tl = 0; tl < nt; ++tl) {
      ls += lsq[tl];
      hs += hsq[tl];
    }
    lpart[blk] = ls;
    hpart[blk] = hs;
  }
}

// ------------------------------------------------------------------------------------------
// Per-token routing of a 64-token block by all eight waves (many experts): lane l owns token l
// and wave w a slice of the experts, so every lane works. Each wave forms its slice's partial
// maximum and exp-sum (combined over the waves in wave order, so lse is the same in every wave and
// reproducible), writes g back over its logits and keeps a sorted top-KM list of its slice. The
// lists then merge pairwise in three rounds through LDS: the list of the lower expert range takes
// the other's entries by strict-greater insertion, so equal scores still go to the lower expert
// index and the merged order is the one a single walk over all experts gives. Wave 0 ends with
// every token's list and writes the gates. Same outputs and partials as route_tokens.
//   L: [64][Ls] fp32; part: [8][64] floats; xv/xi: [4][64][KM] exchange lists.
// ------------------------------------------------------------------------------------------
template <int KM>
__device__ void route_tokens_split(float* L, int Ls, int64_t t0, int64_t T, int E, int k,
                                   int flags, const float* __restrict__ b,
                                   int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
                                   int32_t* __restrict__ hist, float* __restrict__ gpart,
                                   float* __restrict__ lpart, float* __restrict__ hpart,
                                   float* __restrict__ cols, int* hcnt, float* lsq, float* hsq,
                                   float* part, float* part2,
                                   float* xv, int* xi) {
  constexpr int TB = 64, NW = 8;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tl = lane;
  const int64_t t = t0 + tl;
  const bool live = t < T;
  const int E4 = (E + 3) & ~3;
  const int SL = ((E4 / 4 + NW - 1) / NW) * 4;  // experts per wave, a multiple of 4
  const int e0 = min(wave * SL, E4), e1 = min(e0 + SL, E4);
  float* row = L + tl * Ls;
  for (int e = threadIdx.x; e < E; e += blockDim.x) hcnt[e] = 0;
  // maximum over the experts: slice partials, combined in wave order
  float m = -INFINITY;
  for (int e = e0; e < e1; e += 4) {
    const float4 v = *reinterpret_cast<const float4*>(row + e);
    m = fmaxf(m, fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)));
  }
  part[wave * TB + tl] = m;
  __syncthreads();
  m = part[tl];
  for (int w = 1; w < NW; ++w) m = fmaxf(m, part[w * TB + tl]);
  float sum = 0.f;
  for (int e = e0; e < e1; e += 4) {
    const float4 v = *reinterpret_cast<const float4*>(row + e);
    sum += expf(v.x - m);
    sum += expf(v.y - m);
    sum += expf(v.z - m);
    sum += expf(v.w - m);
  }
  __syncthreads();  // every wave has read the maxima
  part[wave * TB + tl] = sum;
  __syncthreads();
  sum = 0.f;
  for (int w = 0; w < NW; ++w) sum += part[w * TB + tl];
  const float lse = m + logf(sum);
  // scores of the slice, written back over the logits, and the slice's sorted top-KM
  const bool sig = (flags & kRouteSigmoid) != 0;
  const bool ec = (flags & kRouteExpertChoice) != 0;
  float ssum = 0.f;
  float hacc = 0.f;  // entropy term of the slice: softmax sum g (l - lse); sigmoid sum s ln s
  float tv[KM];
  int ti[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    tv[j] = -INFINITY;
    ti[j] = 0;
  }
  for (int e = e0; e < e1; e += 4) {
    float4 v = *reinterpret_cast<const float4*>(row + e);
    const float l4[4] = {v.x, v.y, v.z, v.w};
    if (sig) {
      v.x = 1.f / (1.f + expf(-v.x));
      v.y = 1.f / (1.f + expf(-v.y));
      v.z = 1.f / (1.f + expf(-v.z));
      v.w = 1.f / (1.f + expf(-v.w));
      ssum += v.x;
      ssum += v.y;
      ssum += v.z;
      ssum += v.w;
    } else {
      v.x = expf(v.x - lse);
      v.y = expf(v.y - lse);
      v.z = expf(v.z - lse);
      v.w = expf(v.w - lse);
    }
    *reinterpret_cast<float4*>(row + e) = v;
    const float g4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int ee = e + q;
      if (ee < E) {
        if (ec) {  // expert choice: columns of logits and scores for the per-expert selection
          if (live) {
            cols[static_cast<int64_t>(ee) * T + t] = l4[q];
            cols[(static_cast<int64_t>(E) + ee) * T + t] = g4[q];
          }
        } else {
          topk_insert<KM>(b != nullptr ? g4[q] + b[ee] : g4[q], ee, tv, ti);
        }
        hacc += sig ? (g4[q] > 0.f ? g4[q] * logf(g4[q]) : 0.f) : g4[q] * (l4[q] - lse);
      }
    }
  }
  // pairwise merges: round r, waves w with w % 2^(r+1) == 0 take the list of wave w + 2^r
  for (int r = 0; r < 3; ++r) {
    const int stride = 1 << r;
    __syncthreads();  // the exchange buffer is free (and, first time, the partials were read)
    const bool sender = (wave & (2 * stride - 1)) == stride;
    const int slot = wave >> (r + 1);  // 0..3 at most
    if (sender) {
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        xv[(slot * TB + tl) * KM + j] = tv[j];
        xi[(slot * TB + tl) * KM + j] = ti[j];
      }
    }
    __syncthreads();
    if ((wave & (2 * stride - 1)) == 0) {
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        const float v = xv[(slot * TB + tl) * KM + j];
        if (v > tv[KM - 1]) topk_insert<KM>(v, xi[(slot * TB + tl) * KM + j], tv, ti);
      }
    }
  }
  // slice partials of the score sum (sigmoid) and of the entropy term, combined in wave order
  part[wave * TB + tl] = ssum;
  part2[wave * TB + tl] = hacc;
  __syncthreads();
  if (wave == 0 && live && !ec) {
    float wsum = 0.f;
#pragma unroll
    for (int j = 0; j < KM; ++j)
      if (j < k) wsum += row[ti[j]];
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      if (j < k) {
        const float gj = row[ti[j]];
        topk_idx[t * k + j] = ti[j];
        topk_w[t * k + j] = (flags & kRouteRenorm) ? gj / wsum : gj;
        atomicAdd(&hcnt[ti[j]], 1);
      }
    }
  }
  float tot = 0.f, htot = 0.f;
  for (int w = 0; w < NW; ++w) {
    tot += part[w * TB + tl];
    htot += part2[w * TB + tl];
  }
  if (wave == 0) {
    lsq[tl] = live ? lse * lse : 0.f;
    hsq[tl] = live ? (sig ? logf(tot) - htot / tot : -htot) : 0.f;
  }
  if (sig) {  // the sigmoid probability statistic normalises by the sum over all experts
    __syncthreads();  // wave 0 has read the raw scores of every slice
    const float inv = 1.f / tot;
    for (int e = e0; e < e1; ++e) row[e] *= inv;
  }
  __syncthreads();
  const int64_t blk = blockIdx.x;
  const int nt = static_cast<int>(min<int64_t>(TB, T - t0));
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    float gs = 0.f;
    for (int q = 0; q < nt; ++q) gs += L[q * Ls + e];
    gpart[blk * E + e] = gs;
    hist[blk * E + e] = hcnt[e];
  }
  if (threadIdx.x == 0) {
    float ls = 0.f, hs = 0.f;
    for (int q = 0; q < nt; ++q) {
      ls += lsq[q];
      hs += hsq[q];
    }
    lpart[blk] = ls;
    hpart[blk] = hs;
  }
}

// the top-k list length used for k (2, 8 or 16 slots)
#define MOE_ROUTE_TOKENS_KM(CALL) \
  do {                            \
    if (k <= 2) {                 \
      CALL(2);                    \
    } else if (k <= 8) {          \
      CALL(8);                    \
    } else {                      \
      CALL(16);                   \
    }                             \
  } while (0)

// logits row stride: a multiple of 4 floats (16-byte reads); with at most 16 lanes walking 16
// rows, the rows' 4-bank groups are all distinct
constexpr int kLogitsStride = MOE_E_MAX + 4;

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

template <int MB, int NEB, int NG>
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
  for (int i = tid; i < TB * 4; i += kRouteThreads) {
    const int e = ((E + 3) & ~3) - 4 + (i & 3);
    if (e >= E) L[(i >> 2) * kLogitsStride + e] = -INFINITY;
  }
  __syncthreads();
#define MOE_CALL(KM) \
  route_tokens<KM>(L, kLogitsStride, TB, t0, T, E, k, flags, b, topk_idx, topk_w, hist, gpart, \
                   lpart, hpart, cols, hcnt, lsq, hsq)
  MOE_ROUTE_TOKENS_KM(MOE_CALL);
#undef MOE_CALL
}

// ------------------------------------------------------------------------------------------
// fp32: logits by sequential FMA over the hidden dimension (one (token, expert) pair per thread).
// ------------------------------------------------------------------------------------------
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
  for (int i = threadIdx.x; i < RT * 4; i += blockDim.x) {
    const int e = ((E + 3) & ~3) - 4 + (i & 3);
    if (e >= E) L[(i >> 2) * kLogitsStride + e] = -INFINITY;
  }
  __syncthreads();
#define MOE_CALL(KM) \
  route_tokens<KM>(L, kLogitsStride, RT, t0, T, E, k, flags, b, topk_idx, topk_w, hist, gpart, \
                   lpart, hpart, cols, hcnt, lsq, hsq)
  MOE_ROUTE_TOKENS_KM(MOE_CALL);
#undef MOE_CALL
}

// ------------------------------------------------------------------------------------------
// bf16 with many experts (E > 16): W_r is shared through LDS. A block owns 64 tokens; its eight
// waves are 4 token blocks of 16 x 2 expert halves and each runs the whole hidden dimension, so
// x is streamed once per block and W_r once per block. The x and W_r k-slices (128 wide where two
// stages fit in 120 KB, else 64: longer contiguous row reads) pass through two LDS stages (rows
// padded by 8 bf16: the 16x16x32 fragment reads are bank-conflict-free) with the next slices
// prefetched into a register ring two deep; one barrier per k-step.
// ------------------------------------------------------------------------------------------
#ifndef MOE_ROUTE_SK
#define MOE_ROUTE_SK 128
#endif
#ifndef MOE_ROUTE_PF
#define MOE_ROUTE_PF 2
#endif
// k per step: MOE_ROUTE_SK where two stages of (64 + 16 NEB) padded rows fit in 120 KB, else 64
template <int NEB>
constexpr int route_sk() {
  return 2 * (64 + 16 * NEB) * (MOE_ROUTE_SK + 8) * 2 <= 120 * 1024 ? MOE_ROUTE_SK : 64;
}

// SPLIT: per-token routing by all waves (route_tokens_split) rather than one lane per token; its
// exchange buffers are only allocated then, so that the other variant keeps two blocks per CU.
template <int NEB, bool SPLIT>
__global__ __launch_bounds__(kRouteThreads) void route_bf16_lds_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ W, const float* __restrict__ b,
    int64_t T, int d, int E, int k, int flags, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, int32_t* __restrict__ hist, float* __restrict__ gpart,
    float* __restrict__ lpart, float* __restrict__ hpart, float* __restrict__ cols) {
  constexpr int TB = 64;
  constexpr int kSK = route_sk<NEB>();  // k per step
  constexpr int kSKP = kSK + 8;         // padded LDS row (bf16 elements)
  constexpr int ROWS = TB + 16 * NEB;                 // x rows then W_r rows of a stage
  constexpr int STAGE = ROWS * kSKP;                  // bf16 elements
  constexpr int CPR = kSK / 8;                        // 16-byte chunks per row of a stage
  constexpr int CH = ROWS * CPR;                      // 16-byte chunks per stage
  constexpr int CPT = (CH + kRouteThreads - 1) / kRouteThreads;
  constexpr int NEBH = (NEB + 1) / 2;                 // expert blocks per wave
  constexpr int kStagesBytes = 2 * STAGE * 2;
  constexpr int kLBytes = TB * kLogitsStride * 4;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kStagesBytes > kLBytes ? kStagesBytes : kLBytes];
  __shared__ int hcnt[MOE_E_MAX];
  __shared__ float lsq[TB];
  __shared__ float hsq[TB];
  __shared__ float part[SPLIT ? 8 * TB : 1];         // per-wave partials of the split routing
  __shared__ float part2[SPLIT ? 8 * TB : 1];
  __shared__ float xv[SPLIT ? 4 * TB * 16 : 1];      // its exchange lists (KM <= 16)
  __shared__ int xi[SPLIT ? 4 * TB * 16 : 1];
  bf16_t* st = reinterpret_cast<bf16_t*>(smem);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tb = wave & 3, eh = wave >> 2;
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
  constexpr int PF = MOE_ROUTE_PF;
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
  for (int i = tid; i < TB * 4; i += kRouteThreads) {
    const int e = ((E + 3) & ~3) - 4 + (i & 3);
    if (e >= E) L[(i >> 2) * kLogitsStride + e] = -INFINITY;
  }
  __syncthreads();
#define MOE_CALL(KM)                                                                           \
  if constexpr (SPLIT)                                                                         \
    route_tokens_split<KM>(L, kLogitsStride, t0, T, E, k, flags, b, topk_idx, topk_w, hist,     \
                           gpart, lpart, hpart, cols, hcnt, lsq, hsq, part, part2, xv, xi);                             \
  else                                                                                         \
    route_tokens<KM>(L, kLogitsStride, TB, t0, T, E, k, flags, b, topk_idx, topk_w, hist, gpart, \
                     lpart, hpart, cols, hcnt, lsq, hsq)
  MOE_ROUTE_TOKENS_KM(MOE_CALL);
#undef MOE_CALL
}

template <int NEB>
hipError_t launch_bf16_lds(hipStream_t st, const void* x, const void* W, const float* b, int64_t T,
                           int d, int E, int k, int flags, int32_t* topk_idx, float* topk_w,
                           int32_t* hist, float* gpart, float* lpart, float* hpart,
                           float* cols) {
  // short lists over at most 128 experts stay one lane per token (cheaper than the merge rounds)
  const dim3 grid(static_cast<unsigned>(cdiv(T, 64)));
  if (NEB <= 8 && k <= 2)
    hipLaunchKernelGGL((route_bf16_lds_kernel<NEB, false>), grid, dim3(kRouteThreads), 0, st,
                       static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(W), b, T, d, E,
                       k, flags, topk_idx, topk_w, hist, gpart, lpart, hpart, cols);
  else
    hipLaunchKernelGGL((route_bf16_lds_kernel<NEB, true>), grid, dim3(kRouteThreads), 0, st,
                       static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(W), b, T, d, E,
                       k, flags, topk_idx, topk_w, hist, gpart, lpart, hpart, cols);
  return hipGetLastError();
}

template <int MB, int NEB, int NG>
hipError_t launch_bf16(hipStream_t st, const void* x, const void* W, const float* b,
                       int64_t T, int d, int E, int k, int flags, int32_t* topk_idx,
                       float* topk_w, int32_t* hist, float* gpart, float* lpart, float* hpart,
                           float* cols) {
  const int64_t nblk = cdiv(T, 16 * MB);
  hipLaunchKernelGGL((route_bf16_kernel<MB, NEB, NG>), dim3(static_cast<unsigned>(nblk)),
                     dim3(kRouteThreads), 0, st,
                     static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(W), b, T, d, E, k,
                     flags, topk_idx, topk_w, hist, gpart, lpart, hpart, cols);
  return hipGetLastError();
}

}  // namespace

int route_block_tokens(int dtype, int E) { return dtype == MOE_F32 ? RT : (E <= 16 ? 16 : 64); }

hipError_t launch_route(int dtype, int64_t T, int d, int E, int k, int flags, const void* x,
                        const void* W_r, const float* b, int32_t* topk_idx, float* topk_w,
                        int32_t* hist, float* gpart, float* lpart, float* hpart,
                        float* cols, hipStream_t st) {
  if (dtype == MOE_F32) {
    const int64_t nblk = cdiv(T, RT);
    hipLaunchKernelGGL(route_f32_kernel, dim3(static_cast<unsigned>(nblk)), dim3(256), 0, st,
                       static_cast<const float*>(x), static_cast<const float*>(W_r), b, T, d, E,
                       k, flags, topk_idx, topk_w, hist, gpart, lpart, hpart, cols);
    return hipGetLastError();
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

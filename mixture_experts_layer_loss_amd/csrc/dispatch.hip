// Dispatch: expert loads, capacity, expert-contiguous placement and row copies
// ("MoE：条件计算与路由" §1 loads n_e and §3 capacity C = ceil(c B k / E); the histogram-then-sort
// placement of the DeepseekV3MoE listing and the demo MoE's per-expert capacity cut on the
// adg.csdn.net notes page, §四).
//
// Placement rule: assignment (t, j) with expert e = S_tj has position p = #{t' < t : e in S_t'};
// it is kept iff there is no capacity or p < C, and then lands in row offsets_e + p. Positions are
// computed without atomics on ordering: a block of 64 tokens builds, per expert, the 64-bit mask of
// its tokens that chose the expert (LDS atomicOr is order-independent), so the in-block rank is a
// popcount of the lower bits; the cross-block part is an exclusive scan of the block histograms
// in block order. The result is identical on every run.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int RT = kRouteTokens;  // 64 tokens per block: one bit each in a 64-bit mask

__device__ __forceinline__ bool valid_expert(int e, int E) { return e >= 0 && e < E; }

__global__ __launch_bounds__(256) void count_kernel(int64_t T, int E, int k,
                                                     const int32_t* __restrict__ topk_idx,
                                                     int32_t* __restrict__ hist) {
  __shared__ int cnt[MOE_E_MAX];
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * RT;
  for (int p = threadIdx.x; p < RT * k; p += blockDim.x) {
    const int64_t t = t0 + p / k;
    if (t < T) {
      const int e = topk_idx[t * k + p % k];
      if (valid_expert(e, E)) atomicAdd(&cnt[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[static_cast<int64_t>(blockIdx.x) * E + e] = cnt[e];
}

// Tiles of a group of `rows` rows in the grouped GEMM's three classes (BM = 256): full 256-row
// tiles, plus a remainder of 129..255 rows as one more 256-row tile, of 65..128 rows as a 128-row
// tile, or of 1..64 rows as a 64-row tile. With any other BM all tiles are BM rows.
__device__ __forceinline__ void tile_counts(int rows, int BM, int& t_main, int& t128, int& t64) {
  if (BM != 256) {
    t_main = (rows + BM - 1) / BM;
    t128 = t64 = 0;
    return;
  }
  const int rem = rows & 255;
  t_main = (rows >> 8) + (rem > 128 ? 1 : 0);
  t128 = (rem > 64 && rem <= 128) ? 1 : 0;
  t64 = (rem > 0 && rem <= 64) ? 1 : 0;
}

// The shared experts' offsets {0, T} and tile tables (one group of all T rows), written by one
// thread: the scan and expert-choice kernels of a layer forward write them, so they take no
// launch of their own.
__device__ __forceinline__ void write_shared_table(int64_t T, int BM, int32_t* __restrict__ offsets,
                                                   int32_t* __restrict__ tile_off) {
  int c0, c1, c2;
  tile_counts(static_cast<int>(T), BM, c0, c1, c2);
  offsets[0] = 0;
  offsets[1] = static_cast<int32_t>(T);
  tile_off[0] = 0;
  tile_off[1] = c0;
  tile_off[2] = 0;
  tile_off[3] = c1;
  tile_off[4] = 0;
  tile_off[5] = c2;
}

// Inclusive scan over 256 ints in LDS (Hillis-Steele); every thread of the block must call it.
__device__ int block_scan_256(int v, int* buf) {
  const int tid = threadIdx.x;
  buf[tid] = v;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int add = tid >= off ? buf[tid - off] : 0;
    __syncthreads();
    buf[tid] += add;
    __syncthreads();
  }
  const int r = buf[tid];
  __syncthreads();
  return r;
}

// One block of 1024 threads. Thread (p, e) owns expert e (< EP, the power of two >= E) and part p
// of the block range; parts are summed, scanned over p in log2(P) rounds and walked again to
// write the per-block bases, so every sum is taken in a fixed order.
__global__ __launch_bounds__(1024) void scan_kernel(
    int64_t T, int E, int64_t C, int nblk, const int32_t* __restrict__ hist,
    const float* __restrict__ gpart, int nblk_g, const float* __restrict__ lpart,
    const float* __restrict__ hpart, int32_t* __restrict__ block_base,
    int32_t* __restrict__ n_out, double* __restrict__ gsum, double* __restrict__ lse2sum,
    double* __restrict__ hsum, int32_t* __restrict__ kept_out, int32_t* __restrict__ overflow,
    int32_t* __restrict__ offsets, int32_t* __restrict__ tile_off, int BM,
    int32_t* __restrict__ sh_offsets, int32_t* __restrict__ sh_tile_off) {
  __shared__ int psum[1024];
  if (sh_offsets != nullptr && threadIdx.x == 0) write_shared_table(T, BM, sh_offsets, sh_tile_off);
  __shared__ double pg[1024];
  __shared__ int wtot[4][4];
  __shared__ double wred[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int EP = 1;
  while (EP < E) EP <<= 1;
  const int P = 1024 / EP;
  const int e = tid % EP, p = tid / EP;
  // load counts over this part's blocks
  const int b0 = static_cast<int>(static_cast<int64_t>(p) * nblk / P);
  const int b1 = static_cast<int>(static_cast<int64_t>(p + 1) * nblk / P);
  // the loops over blocks are unrolled so that many independent loads are in flight at once
  int cnt = 0;
  if (e < E) {
#pragma unroll 16
    for (int b = b0; b < b1; ++b) cnt += hist[static_cast<int64_t>(b) * E + e];
  }
  psum[tid] = cnt;
  // sum of g over this part's (router) blocks
  double gs = 0.0;
  if (gpart != nullptr && e < E) {
    const int g0 = static_cast<int>(static_cast<int64_t>(p) * nblk_g / P);
    const int g1 = static_cast<int>(static_cast<int64_t>(p + 1) * nblk_g / P);
#pragma unroll 16
    for (int b = g0; b < g1; ++b) gs += static_cast<double>(gpart[static_cast<int64_t>(b) * E + e]);
  }
  pg[tid] = gs;
  __syncthreads();
  // over the parts of each expert, in log2(P) rounds: an inclusive prefix of the counts
  // (Hillis-Steele) and a pairwise tree sum of g (pairs fixed by the part index: reproducible)
  for (int off = 1; off < P; off <<= 1) {
    const int add = p >= off ? psum[tid - off * EP] : 0;
    const int half = P / (2 * off);
    const double gadd = p < half ? pg[tid + half * EP] : 0.0;
    __syncthreads();
    psum[tid] += add;
    if (p < half) pg[tid] += gadd;
    __syncthreads();
  }
  if (e < E && block_base != nullptr) {
    int base = psum[tid] - cnt;  // the counts of the lower parts
#pragma unroll 16
    for (int b = b0; b < b1; ++b) {
      block_base[static_cast<int64_t>(b) * E + e] = base;
      base += hist[static_cast<int64_t>(b) * E + e];
    }
  }
  // per-expert totals (threads of part 0)
  int n = 0, kept = 0;
  if (p == 0 && e < E) {
    n = psum[(P - 1) * EP + e];
    const double g = pg[e];
    kept = (C < 0 || n <= C) ? n : static_cast<int>(C);
    if (n_out != nullptr) n_out[e] = n;
    if (gsum != nullptr) gsum[e] = g;
    if (kept_out != nullptr) kept_out[e] = kept;
    if (overflow != nullptr) overflow[e] = n - kept;
  }
  // exclusive scans over experts: expert e's totals sit in thread e (part 0 is threads [0, EP)).
  // Four inclusive scans over threads 0..255 at once: within each wave by shuffles, then the
  // totals of the lower waves added.
  const int ee = tid < 256 ? tid : 0;
  const bool mine = tid < E;
  const int kept_e = mine ? kept : 0;
  // grouped-GEMM tile tables: [E+1] 256-row (or BM-row) tiles, [E+1] 128-row, [E+1] 64-row
  int c0 = 0, c1 = 0, c2 = 0;
  if (mine) tile_counts(kept_e, BM, c0, c1, c2);
  int v[4] = {kept_e, c0, c1, c2};
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int t = __shfl_up(v[q], off, 64);
      if (lane >= off) v[q] += t;
    }
  }
  if (lane == 63 && wave < 4) {
#pragma unroll
    for (int q = 0; q < 4; ++q) wtot[wave][q] = v[q];
  }
  __syncthreads();
  if (wave < 4) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      for (int w = 0; w < wave; ++w) v[q] += wtot[w][q];
  }
  const int incl = v[0], i0 = v[1], i1 = v[2], i2 = v[3];
  if (mine && offsets != nullptr) {
    offsets[ee] = incl - kept_e;
    if (ee == E - 1) offsets[E] = incl;
  }
  if (mine && tile_off != nullptr) {
    tile_off[ee] = i0 - c0;
    tile_off[E + 1 + ee] = i1 - c1;
    tile_off[2 * (E + 1) + ee] = i2 - c2;
    if (ee == E - 1) {
      tile_off[E] = i0;
      tile_off[2 * E + 1] = i1;
      tile_off[3 * E + 2] = i2;
    }
  }
  // block sums of lse^2 and of the routing entropy: strided partials, a butterfly in each wave,
  // then the 16 wave sums in order (a fixed order: bit-reproducible)
  auto tree = [&](const float* part, double* out) {
    double ls = 0.0;
    for (int b = tid; b < nblk_g; b += 1024) ls += static_cast<double>(part[b]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ls += __shfl_xor(ls, off, 64);
    if (lane == 0) wred[wave] = ls;
    __syncthreads();
    if (tid == 0) {
      double t = 0.0;
      for (int w = 0; w < 16; ++w) t += wred[w];
      *out = t;
    }
    __syncthreads();
  };
  if (lse2sum != nullptr) tree(lpart, lse2sum);
  if (hsum != nullptr) tree(hpart, hsum);
}

// Ranks and rows of one block of 64 tokens: inv_perm [T,k] and perm_token [rows].
// block_base rows are per histogram block of 64 / base_sub tokens: this 64-token block starts at
// histogram block blk * base_sub.
__global__ __launch_bounds__(256) void place_kernel(int64_t T, int E, int k, int64_t C,
                                                     const int32_t* __restrict__ topk_idx,
                                                     int base_sub,
                                                     const int32_t* __restrict__ block_base,
                                                     const int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ perm_token,
                                                     int32_t* __restrict__ inv_perm) {
  __shared__ unsigned int mask[MOE_E_MAX * 2];  // per expert: tokens 0..31, tokens 32..63
  for (int i = threadIdx.x; i < 2 * E; i += blockDim.x) mask[i] = 0u;
  __syncthreads();
  const int64_t blk = blockIdx.x;
  const int64_t t0 = blk * RT;
  for (int p = threadIdx.x; p < RT * k; p += blockDim.x) {
    const int tl = p / k;
    const int64_t t = t0 + tl;
    if (t < T) {
      const int e = topk_idx[t * k + p % k];
      if (valid_expert(e, E)) atomicOr(&mask[2 * e + (tl >> 5)], 1u << (tl & 31));
    }
  }
  __syncthreads();
  for (int p = threadIdx.x; p < RT * k; p += blockDim.x) {
    const int tl = p / k, j = p % k;
    const int64_t t = t0 + tl;
    if (t >= T) continue;
    const int e = topk_idx[t * k + j];
    int row = -1;
    if (valid_expert(e, E)) {
      const unsigned long long m =
          (static_cast<unsigned long long>(mask[2 * e + 1]) << 32) | mask[2 * e];
      const unsigned long long lower = tl == 0 ? 0ull : (m & ((1ull << tl) - 1ull));
      const int64_t pos = static_cast<int64_t>(block_base[blk * base_sub * E + e]) + __popcll(lower);
      if (C < 0 || pos < C) {
        row = offsets[e] + static_cast<int>(pos);
        perm_token[row] = static_cast<int32_t>(t);
      }
    }
    inv_perm[t * k + j] = row;
  }
}

// x_perm[inv_perm[t, j]] = x[t]: one wave per token, 16-byte chunks, read once, written k times.
__global__ __launch_bounds__(256) void copy_rows_kernel(int64_t T, int k, int64_t row_chunks,
                                                         const uint4* __restrict__ x,
                                                         const int32_t* __restrict__ inv_perm,
                                                         uint4* __restrict__ x_perm) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int rows[MOE_K_MAX];
#pragma unroll
  for (int j = 0; j < MOE_K_MAX; ++j) rows[j] = j < k ? inv_perm[t * k + j] : -1;
  const uint4* src = x + t * row_chunks;
  for (int64_t c = lane; c < row_chunks; c += 64) {
    const uint4 v = src[c];
#pragma unroll
    for (int j = 0; j < MOE_K_MAX; ++j)
      if (rows[j] >= 0) x_perm[static_cast<int64_t>(rows[j]) * row_chunks + c] = v;
  }
}

__global__ __launch_bounds__(256) void schedule_kernel(int groups, const int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ tile_off, int BM,
                                                        int min_tiles) {
  __shared__ int sbuf[256];
  const int g = threadIdx.x;
  const int rows = g < groups ? offsets[g + 1] - offsets[g] : 0;
  int c0 = 0, c1 = 0, c2 = 0;
  if (g < groups && rows > 0) tile_counts(rows, BM, c0, c1, c2);
  if (g < groups) c0 = max(c0, min_tiles);
  const int i0 = block_scan_256(c0, sbuf);
  const int i1 = block_scan_256(c1, sbuf);
  const int i2 = block_scan_256(c2, sbuf);
  if (g < groups) {
    tile_off[g] = i0 - c0;
    tile_off[groups + 1 + g] = i1 - c1;
    tile_off[2 * (groups + 1) + g] = i2 - c2;
    if (g == groups - 1) {
      tile_off[groups] = i0;
      tile_off[2 * groups + 1] = i1;
      tile_off[3 * groups + 2] = i2;
    }
  }
}

// Tile tables of the shared experts: one group of all T rows.
__global__ void shared_table_kernel(int64_t T, int BM, int32_t* __restrict__ offsets,
                                    int32_t* __restrict__ tile_off) {
  if (threadIdx.x == 0) write_shared_table(T, BM, offsets, tile_off);
}

// Offsets of ks row ranges over T rows, cut at multiples of 64 rows: [0, c, 2c, .., T] with
// c = 64 ceil(T / (64 ks)) (a range may be empty).
__global__ void row_splits_kernel(int64_t T, int ks, int32_t* __restrict__ offsets) {
  const int i = threadIdx.x;
  if (i <= ks) {
    const int64_t c = ((T + 64 * ks - 1) / (64 * ks)) * 64;
    offsets[i] = static_cast<int32_t>(i == ks ? T : (i * c < T ? i * c : T));
  }
}

// ------------------------------------------------------------------------------------------
// Expert-choice selection ("深入理解 MoE (混合专家模型)：稀疏激活与高效扩展" §9.2: every expert
// picks its top tokens by its score column; "MoE：条件计算与路由" §路由机制的演进): one block per
// expert takes the r tokens of largest logit, equal logits to the lower token index, and lays
// them out in ascending token order at rows [e r, (e + 1) r).
//   Keys are the logits as order-preserving uint32 (ec_select_kernel below has the steps).
//   lcol [E][T] logits; perm_token [E r]; row_of [E][T] (row or -1); offsets [E+1]; counts,
//   overflow [E]; tile_off [3 (E+1)]: the grouped GEMMs' tile tables for BM-row tiles.
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t order_key(float v) {
  if (v == 0.f) v = 0.f;  // -0 and +0 compare equal: one key
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// inclusive prefix sum of v over the 64 lanes of a wave
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(v, off, 64);
    if (lane >= off) v += y;
  }
  return v;
}

// exclusive prefix sum of v over the 1024 threads of the block, and the block total; wave 0 scans
// the 16 wave totals (wsum: 17 ints of LDS, free again on return)
__device__ __forceinline__ int block_excl_scan(int v, int* wsum, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int x = wave_incl_scan(v);
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  if (wave == 0) {
    const int w = lane < 16 ? wsum[lane] : 0;
    const int wi = wave_incl_scan(w);
    if (lane < 16) wsum[lane] = wi - w;
    if (lane == 15) wsum[16] = wi;
  }
  __syncthreads();
  const int r = wsum[wave] + x - v;
  total = wsum[16];
  __syncthreads();
  return r;
}

// The r-th largest key by a 4-pass MSB-first radix select (8 bits a pass): each wave counts into
// its own LDS histogram (the keys of a column share their top bits, so one shared histogram made
// every atomic of a pass queue on a few addresses), the 16 counts of a bin are summed by one of
// 256 threads, and a scan over the bins from the top finds the bin holding the r-th key. Then the
// column is walked in chunks of 1024 x 8 tokens, 8 consecutive tokens per thread, with two block
// scans per chunk: the rank among keys equal to the threshold (ties: the lowest indices are taken)
// and the row of each taken token.
// The scan kernel's reductions of the router's per-block statistics partials, by a block of 1024
// threads (every thread calls it), in the same order: thread (p, e) sums g of expert e over part p
// of the blocks, the parts are added in a pairwise tree, and lse^2 and entropy are strided sums
// over the threads, a butterfly in each wave and the 16 wave sums in order. pg: 1024 doubles of
// LDS, wred: 16.
__device__ void reduce_route_partials(int E, int nblk_g, const float* __restrict__ gpart,
                                      const float* __restrict__ lpart,
                                      const float* __restrict__ hpart, double* __restrict__ gsum,
                                      double* __restrict__ lse2sum, double* __restrict__ hsum,
                                      double* pg, double* wred) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int EP = 1;
  while (EP < E) EP <<= 1;
  const int P = 1024 / EP;
  const int e = tid % EP, p = tid / EP;
  double gs = 0.0;
  if (e < E) {
    const int g0 = static_cast<int>(static_cast<int64_t>(p) * nblk_g / P);
    const int g1 = static_cast<int>(static_cast<int64_t>(p + 1) * nblk_g / P);
#pragma unroll 16
    for (int b = g0; b < g1; ++b) gs += static_cast<double>(gpart[static_cast<int64_t>(b) * E + e]);
  }
  pg[tid] = gs;
  __syncthreads();
  for (int off = 1; off < P; off <<= 1) {
    const int half = P / (2 * off);
    const double gadd = p < half ? pg[tid + half * EP] : 0.0;
    __syncthreads();
    if (p < half) pg[tid] += gadd;
    __syncthreads();
  }
  if (p == 0 && e < E) gsum[e] = pg[tid];
  auto tree = [&](const float* part, double* out) {
    double ls = 0.0;
    for (int b = tid; b < nblk_g; b += 1024) ls += static_cast<double>(part[b]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ls += __shfl_xor(ls, off, 64);
    if (lane == 0) wred[wave] = ls;
    __syncthreads();
    if (tid == 0) {
      double t = 0.0;
      for (int w = 0; w < 16; ++w) t += wred[w];
      *out = t;
    }
    __syncthreads();
  };
  tree(lpart, lse2sum);
  if (hsum != nullptr) tree(hpart, hsum);
}

// Blocks 0..E-1 select; with the router's statistics partials given (gpart non-null), block E
// reduces them meanwhile (reduce_route_partials), on a CU the E selecting blocks leave free.
__global__ __launch_bounds__(1024) void ec_select_kernel(int64_t T, int E, int r,
                                                          const float* __restrict__ lcol,
                                                          int32_t* __restrict__ perm_token,
                                                          int32_t* __restrict__ row_of,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ overflow,
                                                          int32_t* __restrict__ tile_off, int BM,
                                                          RoutePartials rp,
                                                          int32_t* __restrict__ sh_offsets,
                                                          int32_t* __restrict__ sh_tile_off) {
  __shared__ __attribute__((aligned(16))) int hist[16][256];
  __shared__ int wsum[17];
  __shared__ int sel[2];
  __shared__ double wred[16];
  if (sh_offsets != nullptr && blockIdx.x == 0 && threadIdx.x == 0)
    write_shared_table(T, BM, sh_offsets, sh_tile_off);
  if (static_cast<int>(blockIdx.x) == E) {  // (hist is free in this block: pg in its 16 KB)
    reduce_route_partials(E, rp.nblk, rp.gpart, rp.lpart, rp.hpart, rp.gsum, rp.lse2sum, rp.hsum,
                          reinterpret_cast<double*>(&hist[0][0]), wred);
    return;
  }
  const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* col = lcol + static_cast<int64_t>(e) * T;
  // up to 1024 KPT tokens (one chunk of the final walk below), each thread's KPT consecutive keys
  // are read once and kept in registers through the four histogram passes and that walk
  constexpr int KPT = 8;
  const bool in_regs = T <= 1024 * KPT;
  uint32_t rkey[KPT];
  if (in_regs) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int64_t t = static_cast<int64_t>(tid) * KPT + i;
      rkey[i] = t < T ? order_key(col[t]) : 0u;
    }
  }
  uint32_t prefix = 0, pmask = 0;
  int remaining = r;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 16 * 256; i += 1024) hist[i >> 8][i & 255] = 0;
    __syncthreads();
    if (in_regs) {
#pragma unroll
      for (int i = 0; i < KPT; ++i)
        if (static_cast<int64_t>(tid) * KPT + i < T && (rkey[i] & pmask) == prefix)
          atomicAdd(&hist[wave][(rkey[i] >> shift) & 255u], 1);
    } else {
      for (int64_t t = tid; t < T; t += 1024) {
        const uint32_t key = order_key(col[t]);
        if ((key & pmask) == prefix) atomicAdd(&hist[wave][(key >> shift) & 255u], 1);
      }
    }
    __syncthreads();
    // thread j < 256 holds bin 255 - j; the keys in the bins above it are its exclusive prefix
    int c = 0, incl = 0;
    if (tid < 256) {
#pragma unroll
      for (int w = 0; w < 16; ++w) c += hist[w][255 - tid];
      incl = wave_incl_scan(c);
      if (lane == 63) wsum[wave] = incl;
    }
    __syncthreads();
    if (tid < 256) {
      int base = 0;
      for (int w = 0; w < wave; ++w) base += wsum[w];
      const int bin = 255 - tid, above = base + incl - c;
      // the bin where the count from the top reaches `remaining` (bin 0 if none does)
      if ((remaining <= base + incl || bin == 0) && (above < remaining || bin == 255)) {
        sel[0] = bin;
        sel[1] = remaining - above;
      }
    }
    __syncthreads();
    prefix |= static_cast<uint32_t>(sel[0]) << shift;
    pmask |= 255u << shift;
    remaining = sel[1];
    __syncthreads();
  }
  // prefix is the threshold key; `remaining` tokens equal to it are taken, lowest indices first
  int eq_carry = 0, row_carry = 0;
  for (int64_t base = 0; base < T; base += 1024 * KPT) {
    const int64_t t0 = base + static_cast<int64_t>(tid) * KPT;
    uint32_t key[KPT];
    int neq = 0;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      key[i] = in_regs ? rkey[i] : (t0 + i < T ? order_key(col[t0 + i]) : 0u);
      neq += (t0 + i < T && key[i] == prefix) ? 1 : 0;
    }
    int eq_tot = 0;
    int eq_rank = eq_carry + block_excl_scan(neq, wsum, eq_tot);
    int take_mask = 0, ntake = 0;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      if (t0 + i < T) {
        const bool eq = key[i] == prefix;
        if (key[i] > prefix || (eq && eq_rank < remaining)) {
          take_mask |= 1 << i;
          ++ntake;
        }
        eq_rank += eq ? 1 : 0;
      }
    }
    int take_tot = 0;
    int row = row_carry + block_excl_scan(ntake, wsum, take_tot);
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      if (t0 + i < T) {
        const bool take = (take_mask >> i) & 1;
        const bool kept = take && row < r;  // exactly r are taken; the bound guards the row buffer
        const int out = kept ? e * r + row : -1;
        row_of[static_cast<int64_t>(e) * T + t0 + i] = out;
        if (kept) perm_token[out] = static_cast<int32_t>(t0 + i);
        row += take ? 1 : 0;
      }
    }
    eq_carry += eq_tot;
    row_carry += take_tot;
  }
  if (tid == 0) {
    offsets[e] = e * r;
    if (e == E - 1) offsets[E] = E * r;
    counts[e] = r;
    overflow[e] = 0;
    // the grouped GEMMs' tile tables: every expert has r rows, so its tiles of each class are
    // e times one expert's
    int c0 = 0, c1 = 0, c2 = 0;
    if (r > 0) tile_counts(r, BM, c0, c1, c2);
    tile_off[e] = e * c0;
    tile_off[E + 1 + e] = e * c1;
    tile_off[2 * (E + 1) + e] = e * c2;
    if (e == E - 1) {
      tile_off[E] = E * c0;
      tile_off[2 * E + 1] = E * c1;
      tile_off[3 * E + 2] = E * c2;
    }
  }
}

}  // namespace

hipError_t launch_ec_select(int64_t T, int E, int r, const float* lcol, int32_t* perm_token,
                            int32_t* row_of, int32_t* offsets, int32_t* counts,
                            int32_t* overflow, int32_t* tile_off, int BM, hipStream_t st,
                            const RoutePartials* rp, int32_t* sh_offsets, int32_t* sh_tile_off) {
  const RoutePartials none{};
  const bool red = rp != nullptr && rp->gpart != nullptr;
  hipLaunchKernelGGL(ec_select_kernel, dim3(E + (red ? 1 : 0)), dim3(1024), 0, st, T, E, r, lcol,
                     perm_token, row_of, offsets, counts, overflow, tile_off, BM,
                     red ? *rp : none, sh_offsets, sh_tile_off);
  return hipGetLastError();
}

hipError_t launch_row_splits(int64_t T, int ks, int32_t* offsets, hipStream_t st) {
  hipLaunchKernelGGL(row_splits_kernel, dim3(1), dim3(64), 0, st, T, ks, offsets);
  return hipGetLastError();
}

hipError_t launch_shared_table(
int64_t T, int BM, int32_t* offsets, int32_t* tile_off,
                               hipStream_t st) {
  hipLaunchKernelGGL(shared_table_kernel, dim3(1), dim3(64), 0, st, T, BM, offsets, tile_off);
  return hipGetLastError();
}

hipError_t launch_count(int64_t T, int E, int k, const int32_t* topk_idx, int32_t* hist,
                        hipStream_t st) {
  hipLaunchKernelGGL(count_kernel, dim3(static_cast<unsigned>(cdiv(T, RT))), dim3(256), 0, st, T,
                     E, k, topk_idx, hist);
  return hipGetLastError();
}

hipError_t launch_scan(int64_t T, int E, int64_t C, int nblk, const int32_t* hist,
                       const float* gpart, const float* lpart, const float* hpart,
                       int32_t* block_base, int32_t* n_out, double* gsum, double* lse2sum,
                       double* hsum, int32_t* kept, int32_t* overflow, int32_t* offsets,
                       int32_t* tile_off, int BM, hipStream_t st, int32_t* sh_offsets,
                       int32_t* sh_tile_off) {
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, st, T, E, C, nblk, hist, gpart, nblk,
                     lpart, hpart, block_base, n_out, gsum, lse2sum, hsum, kept, overflow, offsets,
                     tile_off, BM, sh_offsets, sh_tile_off);
  return hipGetLastError();
}

hipError_t launch_scatter(int64_t T, int d, int E, int k, int64_t C, int elem_bytes,
                          const void* x, const int32_t* topk_idx, int hist_block_tokens,
                          const int32_t* block_base, const int32_t* offsets, void* x_perm,
                          int32_t* perm_token, int32_t* inv_perm, hipStream_t st) {
  hipLaunchKernelGGL(place_kernel, dim3(static_cast<unsigned>(cdiv(T, RT))), dim3(256), 0, st, T,
                     E, k, C, topk_idx, RT / hist_block_tokens, block_base, offsets, perm_token,
                     inv_perm);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || x_perm == nullptr) return err;
  const int64_t row_chunks = static_cast<int64_t>(d) * elem_bytes / 16;
  hipLaunchKernelGGL(copy_rows_kernel, dim3(static_cast<unsigned>(cdiv(T, 4))), dim3(256), 0, st,
                     T, k, row_chunks, static_cast<const uint4*>(x), inv_perm,
                     static_cast<uint4*>(x_perm));
  return hipGetLastError();
}

hipError_t launch_schedule(int groups, const int32_t* offsets, int32_t* tile_off, int BM,
                           hipStream_t st, int min_tiles) {
  if (groups > 256 || (min_tiles > 0 && BM == 256)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(256), 0, st, groups, offsets, tile_off, BM,
                     min_tiles);
  return hipGetLastError();
}

}  // namespace moe

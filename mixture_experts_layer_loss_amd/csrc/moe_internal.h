// Internal declarations shared by the HIP translation units of the MoE layer library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// ------------------------------------------------------------------------------ tiling constants
constexpr int kRouteTokens = 64;   // tokens per route / dispatch block (one bit per token in a u64)
constexpr int kGemmBM = 256;       // rows per grouped-GEMM tile (bf16 path)
constexpr int kGemmF32BM = 64;     // rows per grouped-GEMM tile (fp32 path)

// ------------------------------------------------------------------------------ element helpers
typedef uint16_t bf16_t;  // raw bf16 bits

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// fp32 -> bf16, round to nearest, ties to even (gfx950 converts in hardware: v_cvt_pk_bf16_f32);
// NaN stays a NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ __forceinline__ static float load(const float* p, int64_t i) { return p[i]; }
  __device__ __forceinline__ static float to_f32(float v) { return v; }
  __device__ __forceinline__ static float from_f32(float v) { return v; }
};
template <> struct Elem<bf16_t> {
  __device__ __forceinline__ static float to_f32(bf16_t v) { return bf16_to_f32(v); }
  __device__ __forceinline__ static bf16_t from_f32(float v) { return f32_to_bf16(v); }
};

__host__ __device__ inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ------------------------------------------------------------------------------ launchers
// Each returns hipSuccess or the launch error; all enqueue on `st`.

// Tokens per router block: the router writes its partial statistics and expert histogram per
// block of this many tokens (a divisor of kRouteTokens).
int route_block_tokens(int dtype, int E, int64_t T);

// Router flags: renormalise the chosen gates; score the experts with a sigmoid (else softmax);
// expert choice (no per-token top-k: the logits and scores leave as [E][T] columns instead).
constexpr int kRouteRenorm = 1, kRouteSigmoid = 2, kRouteExpertChoice = 4;

// Router: logits, softmax/LSE, biased top-k, gates, per-block partial statistics and histograms.
//   hist  [nblk, E] int32, gpart [nblk, E] fp32, lpart [nblk] fp32 (sum of lse^2),
//   hpart [nblk] fp32 (sum of the per-token routing entropies), nblk = ceil(T / route_block_tokens)
//   cols [2][E][T] fp32 (expert choice only, else NULL): logits, then scores, expert-major
hipError_t launch_route(int dtype, int64_t T, int d, int E, int k, int flags, const void* x,
                        const void* W_r, const float* b, int32_t* topk_idx, float* topk_w,
                        int32_t* hist, float* gpart, float* lpart, float* hpart, float* cols,
                        hipStream_t st);

// Per-block expert histograms of a given selection (for a stand-alone dispatch).
hipError_t launch_count(int64_t T, int E, int k, const int32_t* topk_idx, int32_t* hist,
                        hipStream_t st);

// One block: reduces the per-block partials (fp64, fixed order), scans loads over blocks, applies
// the capacity and builds offsets and the grouped-GEMM tile table.
//   block_base [nblk, E]; gsum/lse2sum/hsum/gpart/lpart/hpart may be NULL (dispatch-only use).
//   tile_off [3 (E+1)]: grouped-GEMM tile tables (exclusive prefixes over groups) of 256-row,
//   128-row and 64-row tiles when BM = 256, else of BM-row tiles and two zero tables.
//   sh_offsets [2], sh_tile_off [6]: NULL, or where to write the shared experts' offsets and tile
//   tables as launch_shared_table does.
hipError_t launch_scan(int64_t T, int E, int64_t C, int nblk, const int32_t* hist,
                       const float* gpart, const float* lpart, const float* hpart,
                       int32_t* block_base, int32_t* n_out, double* gsum, double* lse2sum,
                       double* hsum, int32_t* kept, int32_t* overflow, int32_t* offsets,
                       int32_t* tile_off, int BM, hipStream_t st, int32_t* sh_offsets = nullptr,
                       int32_t* sh_tile_off = nullptr);

// Places assignments: inv_perm, perm_token and (when x_perm != NULL) the x row copies.
// block_base holds one row per histogram block of hist_block_tokens tokens (a divisor of
// kRouteTokens).
hipError_t launch_scatter(int64_t T, int d, int E, int k, int64_t C, int elem_bytes,
                          const void* x, const int32_t* topk_idx, int hist_block_tokens,
                          const int32_t* block_base, const int32_t* offsets, void* x_perm,
                          int32_t* perm_token, int32_t* inv_perm, hipStream_t st);

// Expert-choice selection: expert e takes the r tokens of largest lcol[e][t] (ties: lower t) at
// rows e r .. e r + r - 1 in ascending token order; row_of [E][T] = row or -1; offsets [E+1] = e r;
// counts = r, overflow = 0; tile_off: the grouped GEMMs' tile tables for BM-row tiles (as
// launch_schedule writes them for these offsets).
// The router's per-block statistics partials (gpart [nblk][E], lpart and hpart [nblk]) and where
// their reductions go (as the scan kernel computes them; hpart / hsum may be NULL).
struct RoutePartials {
  const float* gpart;
  const float* lpart;
  const float* hpart;
  int nblk;
  double* gsum;
  double* lse2sum;
  double* hsum;
};
// rp: NULL, or partials to reduce in an extra block of the same launch. sh_offsets, sh_tile_off:
// as for launch_scan.
hipError_t launch_ec_select(int64_t T, int E, int r, const float* lcol, int32_t* perm_token,
                            int32_t* row_of, int32_t* offsets, int32_t* counts,
                            int32_t* overflow, int32_t* tile_off, int BM, hipStream_t st,
                            const RoutePartials* rp = nullptr, int32_t* sh_offsets = nullptr,
                            int32_t* sh_tile_off = nullptr);

// The inputs and outputs of the balance statistics (launch_stats below), for a combine launch to
// compute them in one extra block beside its own blocks.
struct StatsArgs {
  int64_t T;
  int E;
  double fden;
  const int32_t* n;
  const double* gsum;
  const double* lse2sum;
  const double* hsum;
  float lambda;
  float* f;
  float* P;
  float* aux;
  float* z;
  float* diag;
  const float* b;
  float* b_new;
  float gamma;
};

// Expert-choice combine: y_t = sum over experts e (ascending) with row_of[e][t] >= 0 of
// w_te out_perm[row] + shared_t, w_te = gcol[e][t] (renormalised over those experts if renorm).
// stats: NULL, or the balance statistics to compute in the same launch.
hipError_t launch_combine_ec(int dtype, int64_t T, int d, int E, int renorm, const void* out_perm,
                             const int32_t* row_of, const float* gcol, const void* shared_out,
                             void* y, hipStream_t st, const StatsArgs* stats = nullptr);

// Tile tables [3 (groups+1)] of a grouped GEMM from device row offsets (stand-alone expert FFN).
// min_tiles > 0 (BM != 256 only): every group, empty ones included, gets at least that many tiles
// in the first table (the weight gradients' zero-padded column ranges).
hipError_t launch_schedule(int groups, const int32_t* offsets, int32_t* tile_off, int BM,
                           hipStream_t st, int min_tiles = 0);

// Grouped SwiGLU FFN in two launches. max_tiles = upper bound of sum_g ceil(rows_g / BM).
//   gate/up: h[r] = SiLU(a_r W_gate[g]^T) * (a_r W_up[g]^T), a_r = rows[r], or rows[gather[r]]
//            when gather != NULL (rows is then the token matrix)
//   down:    out[r] = h[r] W_down[g]^T
// a_rows: rows of the matrix the product reads (rows, or h), which lets the bf16 kernels address
// it with 32-bit offsets when it spans less than 4 GiB.
hipError_t launch_gemm_up(int dtype, int groups, int d, int Mg, const void* rows,
                          const int32_t* gather, const int32_t* offsets, const int32_t* tile_off,
                          int64_t max_tiles, const void* W_gate, const void* W_up, void* h,
                          hipStream_t st, int64_t a_rows);
// part: NULL, or [2][groups][128][d] fp32 in which a bf16 product too long for the persistent
// kernel computes its remainder tiles (1..128 rows past each group's 256-row tiles) in two K chunks
hipError_t launch_gemm_down(int dtype, int groups, int d, int Mg, const int32_t* offsets,
                            const int32_t* tile_off, int64_t max_tiles, const void* W_down,
                            const void* h, void* out, hipStream_t st, int64_t a_rows,
                            float* part = nullptr);

// Gradient of aux + z_coef z with respect to the logits, from the router's logit and score
// columns [E][T]; n [E] loads, fden the f_e denominator. dl [T][E] and dlT [E][T] fp32.
hipError_t launch_loss_grad(int64_t T, int E, int sigmoid, const float* lcol, const float* scol,
                            const int32_t* n, double fden, float lambda, float z_coef, float* dl,
                            float* dlT, hipStream_t st);
// C[M][N] fp32 = sum_k A[k][m] B[k][n]; A fp32 [K][M], B [K][N] of dtype_b (bf16 or fp32). K is
// split into KS ranges (kmajor_splits) whose partials (KS M N floats of `partial`, unused when
// KS = 1) are summed in range order.
int kmajor_splits(int64_t M, int64_t N, int64_t K);
hipError_t launch_kmajor_gemm(int dtype_b, int64_t M, int64_t N, int64_t K, int KS, const float* A,
                              const void* B, float* C, float* partial, hipStream_t st);

// Plain grouped GEMM C[r] = A_r B_g^T (A_r = rows[gather[r]] when gather != NULL), dtype in,
// fp32 out.
hipError_t launch_gemm_plain(int dtype, int groups, const void* rows, const int32_t* gather,
                             const int32_t* offsets, const int32_t* tile_off, int64_t max_tiles,
                             const void* B, int64_t group_stride, int N, int K, void* C,
                             hipStream_t st);

// Backward (backward.hip). Per kept row, from P = dy_t W_down[e] and the fp32 pre-activations:
// dw [T, k] (slot of the row) and the SwiGLU derivative of dh = w P, as fp32 dG, dU [R, M] or, when
// dGU != NULL, one bf16 row [dG | dU] of 2M; when not NULL wh [R, M] bf16 = w SiLU(G) U,
// dout = w dy_t and wrow = w.
hipError_t launch_bw_rows(int dtype, const int32_t* offsets, int E, int64_t R, int d, int M,
                          int k, const int32_t* perm_token, const int32_t* inv_perm,
                          const float* topk_w, const void* dy, const float* P, const float* G,
                          const float* U, float* dw, float* dG, float* dU, void* dGU, void* wh,
                          float* dout, float* wrow, hipStream_t st);
hipError_t launch_swiglu_fwd(int64_t count, const float* G, const float* U, float* h,
                             hipStream_t st);
hipError_t launch_bw_router(int64_t T, int E, int k, int renorm, int sigmoid, const float* lcol,
                            const float* scol, const int32_t* topk_idx, const int32_t* inv_perm,
                            const float* topk_w, const float* dw, const int32_t* n, double fden,
                            float lambda, float z_coef, float* dl, float* dlT, hipStream_t st);
// C[r][n] (fp32) = sum_k A[a(r)][k] B_g[k][n] (+ A2 B2_g), a(r) = gather_a[r] or r; 64-row tile
// table tile_off per group
hipError_t launch_nn_gemm(int dtype_a, int dtype_b, bool two, const void* A, const void* A2,
                          const int32_t* gather_a, const int32_t* offsets, const int32_t* tile_off,
                          int groups, int64_t max_tiles, const void* B, const void* B2,
                          int64_t gstride, int N, int K, float* C, hipStream_t st);
// C_g[m][n] (fp32, [groups][Ma][Nb]) = sum over rows r of group g of A[r][m] B[b(r)][n]
hipError_t launch_kk_gemm(int dtype_a, int dtype_b, const void* A, int Ma, const void* B, int Nb,
                          const int32_t* gather, const int32_t* offsets, int groups, float* C,
                          hipStream_t st);
hipError_t launch_swiglu_bw(int dtype, int64_t count, const float* dh, const void* G,
                            const void* U, float* dG, float* dU, hipStream_t st);
hipError_t launch_bw_dx(int64_t T, int d, int k, const int32_t* inv_perm, const float* dx_perm,
                        const float* dx_sh, float* dx, hipStream_t st);
// Expert choice (row_of [E][T], scores scol [E][T]): the row gates wrow [R]; the router backward
// from per-row d w; dx_t += the token's dx rows in ascending expert order (+ dx_sh).
hipError_t launch_ec_gates(int64_t T, int E, int renorm, const int32_t* row_of,
                           const float* scol, float* wrow, hipStream_t st);
hipError_t launch_bw_router_ec(int64_t T, int E, int renorm, int sigmoid, const int32_t* row_of,
                               const float* lcol, const float* scol, const float* dw,
                               const int32_t* n, double fden, float lambda, float z_coef,
                               float* dl, float* dlT, hipStream_t st);
hipError_t launch_bw_dx_ec(int64_t T, int d, int E, const int32_t* row_of, const float* dx_perm,
                           const float* dx_sh, float* dx, hipStream_t st);

// bf16 backward on MFMA (backward_layout.hip, gemm_bf16.hip).
// dst [r] (bf16 [rows][d]) = src [gather[r]] for the kept rows r < offsets[groups] (of at most R)
hipError_t launch_gather_rows(const void* src, int d, const int32_t* gather,
                              const int32_t* offsets, int groups, int64_t R, void* dst,
                              hipStream_t st);
// dGU [R][2M] bf16 = [dh U SiLU'(G) | dh SiLU(G)] and h [R][M] bf16 = SiLU(G) U from fp32 [R][M]
hipError_t launch_swiglu_bw_cat(int64_t R, int M, const float* dh, const float* G, const float* U,
                                void* dGU, void* h, hipStream_t st);
// C[r] (fp32) = A_r B_g with B_g [K][N] (N contiguous); with B1, rows K/2.. of B_g come from B1.
// part: NULL, or [2][groups][128][N] fp32 in which the remainder tiles (1..128 rows past each
// group's 256-row tiles) run in two K chunks (with B1: the halves, K/2 a multiple of 64)
hipError_t launch_gemm_kn_bf16(int groups, const void* rows, const int32_t* gather,
                               const int32_t* offsets, const int32_t* tile_off, int64_t max_tiles,
                               const void* B0, const void* B1, int64_t group_stride, int N, int K,
                               float* C, hipStream_t st, float* part = nullptr);
// h as launch_gemm_up_bf16 writes it, plus G and U as launch_gemm_gu_f32out_bf16 writes them
hipError_t launch_gemm_up_save_bf16(int groups, int d, int Mg, const void* rows,
                                    const int32_t* gather, const int32_t* offsets,
                                    const int32_t* tile_off, int64_t max_tiles, const void* W_gate,
                                    const void* W_up, void* h, float* G, float* U,
                                    hipStream_t st, int64_t a_rows);
// G[r] = a_r W_gate[g]^T, U[r] = a_r W_up[g]^T in fp32 (one launch, gate/up tiles paired)
hipError_t launch_gemm_gu_f32out_bf16(int groups, int d, int Mg, const void* rows,
                                      const int32_t* gather, const int32_t* offsets,
                                      const int32_t* tile_off, int64_t max_tiles,
                                      const void* W_gate, const void* W_up, float* G, float* U,
                                      hipStream_t st, int64_t a_rows);
// C_g [Ma][Nb] fp32 = sum over the rows r of group g ([offsets[g], offsets[g+1]) of `rows`) of
// A[r][m] B[r][n], A [rows][lda] and B [rows][ldb] bf16 read in place (Ma, Nb multiples of 8); kt:
// the groups' k-slice prefix from launch_schedule with BM 64 and min_tiles 2
hipError_t launch_gemm_wgrad_bf16(const void* A, int lda, const void* B, int ldb, int64_t rows,
                                  const int32_t* offsets, const int32_t* kt, int groups, int Ma,
                                  int Nb, float* C, hipStream_t st);

// Offsets [ks + 1] of ks row ranges over T rows, cut at multiples of 64 rows (ks <= 63).
hipError_t launch_row_splits(int64_t T, int ks, int32_t* offsets, hipStream_t st);

// C[i] = sum over s = 0..KS-1, in that order, of P[s count + i].
hipError_t launch_sum_ranges(int64_t count, int KS, const float* P, float* C, hipStream_t st);

// Tile table of the shared experts (one group of all T rows).
hipError_t launch_shared_table(int64_t T, int BM, int32_t* offsets, int32_t* tile_off,
                               hipStream_t st);

// y_t = sum_j w_tj out_perm[inv_tj] (+ shared_t). stats: as for launch_combine_ec.
hipError_t launch_combine(int dtype, int64_t T, int d, int k, const void* out_perm,
                          const int32_t* inv_perm, const float* topk_w, const void* shared_out,
                          void* y, hipStream_t st, const StatsArgs* stats = nullptr);

// dst[0, n) = src[0, n), or zeros when src is NULL.
hipError_t launch_copy_f32(const float* src, float* dst, int n, hipStream_t st);

// f, P, aux, z and the bias step from reduced route statistics.
// fden: the f_e denominator (k T; E r for expert choice). diag (may be NULL) [4]: routing entropy
// (hsum / T), load Gini, max/mean load, importance CV^2.
hipError_t launch_stats(int64_t T, int E, double fden, const int32_t* n, const double* gsum,
                        const double* lse2sum, const double* hsum, float lambda, float* f,
                        float* P, float* aux, float* z, float* diag, const float* b, float* b_new,
                        float gamma, hipStream_t st);

}  // namespace moe

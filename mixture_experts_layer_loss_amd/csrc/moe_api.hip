// extern "C" entry points of the MoE layer library: argument checks, workspace planning and the
// launch sequence of each call. Every check runs on the host before anything is enqueued; the
// library allocates nothing and never synchronises.
#include <math.h>
#include <string.h>

#include <mutex>

#include "moe_internal.h"

namespace moe {
hipError_t launch_gemm_up_bf16(int groups, int d, int Mg, const void* rows,
                               const int32_t* gather, const int32_t* offsets,
                               const int32_t* tile_off, int64_t max_tiles, const void* W_gate,
                               const void* W_up, void* h, hipStream_t st, int64_t a_rows);
hipError_t launch_gemm_down_bf16(int groups, int d, int Mg, const int32_t* offsets,
                                 const int32_t* tile_off, int64_t max_tiles, const void* W_down,
                                 const void* h, void* out, hipStream_t st, int64_t a_rows,
                                 float* part);
hipError_t launch_gemm_up_shared_bf16(int groups, int d, int Mg, const void* x,
                                      const int32_t* gather, const int32_t* offsets,
                                      const int32_t* tile_off, int64_t max_tiles,
                                      const void* W_gate, const void* W_up, void* h, int64_t T,
                                      int SMg, const int32_t* sh_offsets,
                                      const int32_t* sh_tile_off, int64_t sh_tiles,
                                      const void* Ws_gate, const void* Ws_up, void* h_sh,
                                      hipStream_t st);
hipError_t launch_gemm_down_shared_bf16(int groups, int d, int Mg, const int32_t* offsets,
                                        const int32_t* tile_off, int64_t max_tiles,
                                        const void* W_down, const void* h, void* out, int64_t R,
                                        int64_t T, int SMg, const int32_t* sh_offsets,
                                        const int32_t* sh_tile_off, int64_t sh_tiles,
                                        const void* Ws_down, const void* h_sh, void* sh,
                                        hipStream_t st, float* part);
hipError_t launch_gemm_up_f32(int groups, int d, int Mg, const void* rows,
                              const int32_t* gather, const int32_t* offsets,
                              const int32_t* tile_off, int64_t max_tiles, const void* W_gate,
                              const void* W_up, void* h, hipStream_t st);
hipError_t launch_gemm_plain_bf16(int groups, const void* rows, const int32_t* gather,
                                  const int32_t* offsets, const int32_t* tile_off,
                                  int64_t max_tiles, const void* B, int64_t group_stride, int N,
                                  int K, void* C, hipStream_t st);
hipError_t launch_gemm_plain_f32(int groups, const void* rows, const int32_t* gather,
                                 const int32_t* offsets, const int32_t* tile_off,
                                 int64_t max_tiles, const void* B, int64_t group_stride, int N,
                                 int K, void* C, hipStream_t st);

hipError_t launch_gemm_plain(int dtype, int groups, const void* rows, const int32_t* gather,
                             const int32_t* offsets, const int32_t* tile_off, int64_t max_tiles,
                             const void* B, int64_t group_stride, int N, int K, void* C,
                             hipStream_t st) {
  return dtype == MOE_F32 ? launch_gemm_plain_f32(groups, rows, gather, offsets, tile_off,
                                                  max_tiles, B, group_stride, N, K, C, st)
                          : launch_gemm_plain_bf16(groups, rows, gather, offsets, tile_off,
                                                   max_tiles, B, group_stride, N, K, C, st);
}

hipError_t launch_gemm_down_f32(int groups, int d, int Mg, const int32_t* offsets,
                                const int32_t* tile_off, int64_t max_tiles, const void* W_down,
                                const void* h, void* out, hipStream_t st);

hipError_t launch_gemm_up(int dtype, int groups, int d, int Mg, const void* rows,
                          const int32_t* gather, const int32_t* offsets, const int32_t* tile_off,
                          int64_t max_tiles, const void* W_gate, const void* W_up, void* h,
                          hipStream_t st, int64_t a_rows) {
  return dtype == MOE_F32
             ? launch_gemm_up_f32(groups, d, Mg, rows, gather, offsets, tile_off, max_tiles,
                                  W_gate, W_up, h, st)
             : launch_gemm_up_bf16(groups, d, Mg, rows, gather, offsets, tile_off, max_tiles,
                                   W_gate, W_up, h, st, a_rows);
}

hipError_t launch_gemm_down(int dtype, int groups, int d, int Mg, const int32_t* offsets,
                            const int32_t* tile_off, int64_t max_tiles, const void* W_down,
                            const void* h, void* out, hipStream_t st, int64_t a_rows,
                            float* part) {
  return dtype == MOE_F32 ? launch_gemm_down_f32(groups, d, Mg, offsets, tile_off, max_tiles,
                                                 W_down, h, out, st)
                          : launch_gemm_down_bf16(groups, d, Mg, offsets, tile_off, max_tiles,
                                                  W_down, h, out, st, a_rows, part);
}
}  // namespace moe

using namespace moe;

namespace {

constexpr size_t kAlign = 256;
// Largest hidden size d, and largest 2 M and 2 S M (the backward's [dG dU] rows), a layer may have.
constexpr int64_t kMaxWidth = int64_t{1} << 21;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int elem_bytes(const moe_shape* s) { return s->dtype == MOE_F32 ? 4 : 2; }
bool expert_choice(const moe_shape* s);
int64_t ec_tokens(const moe_shape* s);
// denominator of f_e: k T assignments (token choice) or E r (expert choice)
double stats_fden(const moe_shape* s) {
  return expert_choice(s) ? static_cast<double>(ec_tokens(s)) * s->E
                          : static_cast<double>(s->k) * static_cast<double>(s->T);
}
int route_flags(const moe_shape* s) {
  return (s->renorm ? kRouteRenorm : 0) | (s->scoring == MOE_SCORE_SIGMOID ? kRouteSigmoid : 0) |
         (s->routing == MOE_ROUTE_EXPERT_CHOICE ? kRouteExpertChoice : 0);
}
int gemm_bm(const moe_shape* s) { return s->dtype == MOE_F32 ? kGemmF32BM : kGemmBM; }
int64_t nblocks(const moe_shape* s) { return cdiv(s->T, kRouteTokens); }
int64_t route_blocks(const moe_shape* s) { return cdiv(s->T, route_block_tokens(s->dtype, s->E, s->T)); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Bump allocator over a caller workspace (or a dry run that only measures).
struct Carve {
  unsigned char* base;
  size_t used = 0;
  explicit Carve(void* b) : base(static_cast<unsigned char*>(b)) {}
  template <typename T>
  T* take(size_t count) {
    T* p = base ? reinterpret_cast<T*>(base + used) : nullptr;
    used += align_up(count * sizeof(T));
    return p;
  }
};

int64_t capacity_of(const moe_shape* s) {
  if (!(s->c > 0.0f)) return -1;
  return static_cast<int64_t>(
      ceil(((static_cast<double>(s->c) * s->k) * static_cast<double>(s->T)) / s->E));
}

bool expert_choice(const moe_shape* s) { return s->routing == MOE_ROUTE_EXPERT_CHOICE; }

// Tokens each expert takes under expert choice: C = ceil(c k T / E), c <= 0 read as 1, at most T.
int64_t ec_tokens(const moe_shape* s) {
  const double c = s->c > 0.0f ? static_cast<double>(s->c) : 1.0;
  const int64_t C = static_cast<int64_t>(ceil(((c * s->k) * static_cast<double>(s->T)) / s->E));
  return C < s->T ? C : s->T;
}

// Rows the routed-expert buffers need: every assignment, or at most C per expert (expert choice:
// exactly r per expert).
int64_t routed_rows(const moe_shape* s) {
  if (expert_choice(s)) return ec_tokens(s) * s->E;
  const int64_t P = s->T * s->k;
  const int64_t C = capacity_of(s);
  return C >= 0 && C * s->E < P ? C * s->E : P;
}

struct RoutePlan {
  int32_t* hist;
  float* gpart;
  float* lpart;
  float* hpart;
};
RoutePlan plan_route(Carve& c, const moe_shape* s) {
  const size_t nb = static_cast<size_t>(route_blocks(s));
  RoutePlan p;
  p.hist = c.take<int32_t>(nb * s->E);
  p.gpart = c.take<float>(nb * s->E);
  p.lpart = c.take<float>(nb);
  p.hpart = c.take<float>(nb);
  return p;
}

struct DispatchPlan {
  int32_t* hist;
  int32_t* block_base;
};
DispatchPlan plan_dispatch(Carve& c, const moe_shape* s) {
  const size_t nb = static_cast<size_t>(nblocks(s));
  DispatchPlan p;
  p.hist = c.take<int32_t>(nb * s->E);
  p.block_base = c.take<int32_t>(nb * s->E);
  return p;
}

struct LayerPlan {
  RoutePlan r;
  int32_t *block_base, *topk_idx, *n, *kept, *overflow, *offsets, *tile_off, *perm_token,
      *inv_perm, *sh_offsets, *sh_tile_off;
  float* topk_w;
  double *gsum, *lse2sum, *hsum;
  void *h, *out_perm, *h_sh, *sh;
  float* cols;      // expert choice: [2][E][T] logits and scores
  int32_t* row_of;  // expert choice: [E][T] row of (t, e) or -1
  float* part;      // [2][E][128][d] fp32 partials of the down product's split remainder tiles
};
LayerPlan plan_layer(Carve& c, const moe_shape* s) {
  const size_t P = static_cast<size_t>(s->T) * s->k;
  const size_t R = static_cast<size_t>(routed_rows(s));
  const size_t eb = static_cast<size_t>(elem_bytes(s));
  LayerPlan p;
  p.r = plan_route(c, s);
  p.block_base = c.take<int32_t>(static_cast<size_t>(route_blocks(s)) * s->E);
  p.topk_idx = c.take<int32_t>(P);
  p.topk_w = c.take<float>(P);
  p.n = c.take<int32_t>(s->E);
  p.gsum = c.take<double>(s->E);
  p.lse2sum = c.take<double>(1);
  p.hsum = c.take<double>(1);
  p.kept = c.take<int32_t>(s->E);
  p.overflow = c.take<int32_t>(s->E);
  p.offsets = c.take<int32_t>(s->E + 1);
  p.tile_off = c.take<int32_t>(3 * (s->E + 1));  // three tile classes of the grouped GEMM
  p.sh_offsets = c.take<int32_t>(2);
  p.sh_tile_off = c.take<int32_t>(3 * 2);
  p.perm_token = c.take<int32_t>(R);
  p.inv_perm = c.take<int32_t>(P);
  p.h = c.take<unsigned char>(R * s->M * eb);
  p.out_perm = c.take<unsigned char>(R * s->d * eb);
  if (s->S > 0) {
    p.h_sh = c.take<unsigned char>(static_cast<size_t>(s->T) * s->S * s->M * eb);
    p.sh = c.take<unsigned char>(static_cast<size_t>(s->T) * s->d * eb);
  } else {
    p.h_sh = p.sh = nullptr;
  }
  if (expert_choice(s)) {
    p.cols = c.take<float>(2 * static_cast<size_t>(s->E) * s->T);
    p.row_of = c.take<int32_t>(static_cast<size_t>(s->E) * s->T);
  } else {
    p.cols = nullptr;
    p.row_of = nullptr;
  }
  p.part = nullptr;
  return p;
}

// Whether the layer forward splits the routed down product's remainder tiles (1..128 rows past
// each expert's 256-row tiles) into two K chunks: bf16 products too long for the persistent kernel
// (M over 128 k-slices), with at least 512 routed rows per expert on average, so that the partial
// buffer stays small next to h.
bool down_split(const moe_shape* s) {
  return s->dtype == MOE_BF16 && s->M > 128 * 64 &&
         routed_rows(s) >= static_cast<int64_t>(512) * s->E;
}

// The partial buffer, carved after everything else of the layer forward's workspace.
float* plan_split(Carve& c, const moe_shape* s) {
  return down_split(s) ? c.take<float>(static_cast<size_t>(2) * s->E * 128 * s->d) : nullptr;
}

struct LossBackwardPlan {
  RoutePlan r;
  float *cols, *dl, *dlT, *partial;
  int ks_w;  // K ranges of the dW_r product
};
LossBackwardPlan plan_loss_backward(Carve& c, const moe_shape* s) {
  const size_t ET = static_cast<size_t>(s->E) * s->T;
  LossBackwardPlan p;
  p.r = plan_route(c, s);
  p.cols = c.take<float>(2 * ET);
  p.dl = c.take<float>(ET);
  p.dlT = c.take<float>(ET);
  p.ks_w = kmajor_splits(s->E, s->d, s->T);
  p.partial = c.take<float>(p.ks_w > 1 ? static_cast<size_t>(p.ks_w) * s->E * s->d : 1);
  return p;
}

// The backward recomputes the forward (LayerPlan) and keeps, per routed row, the gate and up
// pre-activations (fp32; recomputed, or read from the buffer a training forward filled) and the
// fp32 gradients d out, dh, dG, dU and dx_row.
struct LayerBackwardPlan {
  LayerPlan f;
  float* cols;                    // [2][E][T] logits and scores
  int32_t *tile64, *sh_tile64;    // 64-row tile tables of the fp32 products
  float *G, *U;                   // [R, M] fp32 pre-activations
  float *h, *P;                   // [R, M] fp32: SiLU(G) U (fp32 layers) and dy_t W_down[e]
  float *dout, *dw, *dl, *dlT, *dG, *dU, *dxr, *partial;
  int ks_w;
  float *Gs, *Us;                 // shared experts [T, S M] fp32
  float *hs, *dhs, *dGs, *dUs, *dxs;   // [T, S M] and [T, d]
  // bf16 layers (MFMA products): the [dG | dU] rows, and the weight gradients' other row
  // operands: w h per kept row, and the dy and x rows of the kept rows in routed order
  float* wrow;                   // gate of each kept row
  void *dGU, *wh, *dyr, *xr;     // routed experts
  float* part_dx;                // [2][E][128][d]: the dx-row product's split remainder tiles
  void *dGUs, *hsb;              // shared experts: [dGs | dUs] rows and h rows (bf16)
  // the shared experts' weight gradients over ks_sh row ranges of the T rows (bf16 layers): the
  // range offsets, their k-slice table and the ranges' fp32 partials [ks_sh][S M][d]
  int ks_sh;
  int32_t *sh_split_off, *sh_split_kt;
  float* sh_wpart;
};

// Row ranges of the shared experts' weight gradients. Each of the three products has
// ceil(S M / 256) ceil(d / 256) output tiles over all T rows; when those tiles fill under half of
// the chip's 256 compute units, the rows are cut into ks_sh ranges (at least 256 rows each) whose
// partial products run side by side and are summed in range order.
int shared_wgrad_splits(const moe_shape* s) {
  if (s->S <= 0 || s->dtype != MOE_BF16) return 1;
  const int64_t tiles = cdiv(static_cast<int64_t>(s->S) * s->M, 256) * cdiv(s->d, 256);
  int64_t ks = 256 / (tiles > 0 ? tiles : 1);
  ks = ks < 4 ? ks : 4;
  ks = ks < s->T / 256 ? ks : s->T / 256;
  return ks > 1 ? static_cast<int>(ks) : 1;
}
LayerBackwardPlan plan_layer_backward(Carve& c, const moe_shape* s) {
  LayerBackwardPlan p;
  p.f = plan_layer(c, s);
  const size_t R = static_cast<size_t>(routed_rows(s)), T = static_cast<size_t>(s->T);
  const size_t d = s->d, M = s->M, E = s->E;
  p.cols = c.take<float>(2 * E * T);
  p.tile64 = c.take<int32_t>(3 * (E + 1));
  p.sh_tile64 = c.take<int32_t>(3 * 2);
  const bool mfma = s->dtype == MOE_BF16;
  p.G = c.take<float>(R * M);
  p.U = c.take<float>(R * M);
  p.h = mfma ? nullptr : c.take<float>(R * M);
  p.P = c.take<float>(R * M);
  p.dout = mfma ? nullptr : c.take<float>(R * d);
  p.dw = c.take<float>(T * s->k > R ? T * s->k : R);  // per slot, or per row (expert choice)
  p.dl = c.take<float>(T * E);
  p.dlT = c.take<float>(T * E);
  p.dG = mfma ? nullptr : c.take<float>(R * M);
  p.dU = mfma ? nullptr : c.take<float>(R * M);
  p.dxr = c.take<float>(R * d);
  p.wrow = mfma || expert_choice(s) ? c.take<float>(R) : nullptr;
  p.dGU = p.wh = p.dyr = p.xr = nullptr;
  p.dGUs = p.hsb = nullptr;
  p.part_dx = nullptr;
  p.ks_sh = 1;
  p.sh_split_off = p.sh_split_kt = nullptr;
  p.sh_wpart = nullptr;
  if (mfma) {
    p.dGU = c.take<bf16_t>(R * 2 * M);
    p.wh = c.take<bf16_t>(R * M);
    p.dyr = c.take<bf16_t>(R * d);
    p.xr = c.take<bf16_t>(R * d);
    // the dx-row product over K = 2M as for the forward down product: halves of whole k-slices,
    // at least 512 rows per expert
    if (2 * s->M > 128 * 64 && s->M % 64 == 0 && R >= static_cast<size_t>(512) * E)
      p.part_dx = c.take<float>(2 * E * 128 * d);
  }
  p.ks_w = kmajor_splits(s->E, s->d, s->T);
  p.partial = c.take<float>(p.ks_w > 1 ? static_cast<size_t>(p.ks_w) * E * d : 1);
  if (s->S > 0) {
    const size_t SM = static_cast<size_t>(s->S) * M;
    p.Gs = c.take<float>(T * SM);
    p.Us = c.take<float>(T * SM);
    p.hs = mfma ? nullptr : c.take<float>(T * SM);
    p.dhs = c.take<float>(T * SM);
    p.dGs = mfma ? nullptr : c.take<float>(T * SM);
    p.dUs = mfma ? nullptr : c.take<float>(T * SM);
    p.dxs = c.take<float>(T * d);
    if (mfma) {
      p.dGUs = c.take<bf16_t>(T * 2 * SM);
      p.hsb = c.take<bf16_t>(T * SM);
    }
    p.ks_sh = shared_wgrad_splits(s);
    if (p.ks_sh > 1) {
      p.sh_split_off = c.take<int32_t>(p.ks_sh + 1);
      p.sh_split_kt = c.take<int32_t>(3 * (p.ks_sh + 1));
      p.sh_wpart = c.take<float>(static_cast<size_t>(p.ks_sh) * SM * d);
    }
  } else {
    p.Gs = p.Us = nullptr;
    p.hs = p.dhs = p.dGs = p.dUs = p.dxs = nullptr;
  }
  return p;
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Static scratch of moe_layer_forward_noalloc: one copy per device, held until the process ends.
// Host code never uses the array's name as an address (on the host it is only a stand-in): the
// device address comes from hipGetSymbolAddress, once per device, with that device current.
static __device__ __align__(256) unsigned char scratch[MOE_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address (looked up on the first call on that device).
moe_status current_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

// Profiling aid: events recorded at the end of each moe_layer_forward stage (see moe.h). The
// setting is process-wide (the one piece of state the library keeps); it is read and written
// under a lock, and each forward works on the copy it takes when it starts.
std::mutex g_stage_mu;
hipEvent_t g_stage_events[MOE_STAGE_COUNT] = {};
bool g_stage_on = false;

struct StageMarks {
  hipEvent_t ev[MOE_STAGE_COUNT];
  bool on;
  hipError_t err = hipSuccess;  // the first failed record
  StageMarks() {
    std::lock_guard<std::mutex> lock(g_stage_mu);
    on = g_stage_on;
    for (int i = 0; i < MOE_STAGE_COUNT; ++i) ev[i] = g_stage_events[i];
  }
  void mark(int i, hipStream_t st) {
    if (on && ev[i] != nullptr && err == hipSuccess) err = hipEventRecord(ev[i], st);
  }
};

// Pre-activations a training forward keeps for the backward (bf16 layers): the fp32 gate and up
// values of every routed row, [R, M] each with R the workspace's routed-row bound, then those of
// the shared experts, [T, S M] each.
// The bias the forward selected with comes last ([E] fp32, zeros without a bias), so that the
// backward selects exactly as the forward did even if the caller updated b in place in between.
struct SavedPlan {
  float *G, *U, *Gs, *Us, *b;
};
SavedPlan plan_saved(Carve& c, const moe_shape* s) {
  const size_t R = static_cast<size_t>(routed_rows(s)), M = s->M;
  SavedPlan p;
  p.G = c.take<float>(R * M);
  p.U = c.take<float>(R * M);
  if (s->S > 0) {
    const size_t TSM = static_cast<size_t>(s->T) * s->S * M;
    p.Gs = c.take<float>(TSM);
    p.Us = c.take<float>(TSM);
  } else {
    p.Gs = p.Us = nullptr;
  }
  p.b = c.take<float>(s->E);
  return p;
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP launch failed";
    case MOE_ERR_SCRATCH: return "shape needs more than the static scratch of the no-allocation call";
    default: return "unknown status";
  }
}

moe_status moe_check_shape(const moe_shape* s) {
  if (s == nullptr) return MOE_ERR_INVALID_ARGUMENT;
  if (s->dtype != MOE_F32 && s->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (s->T < 1 || s->d < 1 || s->E < 1 || s->k < 1 || s->M < 1 || s->S < 0)
    return MOE_ERR_INVALID_ARGUMENT;
  if (isnan(s->c) || (s->renorm != 0 && s->renorm != 1)) return MOE_ERR_INVALID_ARGUMENT;
  if (s->scoring != MOE_SCORE_SOFTMAX && s->scoring != MOE_SCORE_SIGMOID)
    return MOE_ERR_INVALID_ARGUMENT;
  if (s->routing != MOE_ROUTE_TOKEN_CHOICE && s->routing != MOE_ROUTE_EXPERT_CHOICE)
    return MOE_ERR_INVALID_ARGUMENT;
  if (s->k > s->E) return MOE_ERR_INVALID_ARGUMENT;
  if (s->E > MOE_E_MAX || s->k > MOE_K_MAX) return MOE_ERR_UNSUPPORTED;
  const int vec = s->dtype == MOE_F32 ? 4 : 8;  // elements per 16-byte chunk
  if (s->d % vec != 0 || s->M % vec != 0) return MOE_ERR_INVALID_ARGUMENT;
  // row indices are int32
  if (s->T * static_cast<int64_t>(s->k) > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  if (expert_choice(s) && s->T * static_cast<int64_t>(s->E) > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  // the grouped GEMMs form a tile's operand-row offsets (256 rows of up to 2 max(M, S M) or d
  // elements) in 32 bits
  if (s->d > kMaxWidth || s->M > kMaxWidth / 2 || static_cast<int64_t>(s->S) * s->M > kMaxWidth / 2)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int64_t moe_capacity(const moe_shape* s) {
  if (moe_check_shape(s) != MOE_OK) return -1;
  return capacity_of(s);
}

int64_t moe_routed_rows(const moe_shape* s) {
  if (moe_check_shape(s) != MOE_OK) return -1;
  return routed_rows(s);
}

size_t moe_saved_size(const moe_shape* s) {
  if (moe_check_shape(s) != MOE_OK || s->dtype != MOE_BF16) return 0;
  Carve c(nullptr);
  plan_saved(c, s);
  return c.used;
}

size_t moe_workspace_size(const moe_shape* s, int call) {
  if (moe_check_shape(s) != MOE_OK) return 0;
  Carve c(nullptr);
  switch (call) {
    case MOE_CALL_ROUTE: plan_route(c, s); break;
    case MOE_CALL_DISPATCH: plan_dispatch(c, s); break;
    case MOE_CALL_EXPERT_FFN: c.take<int32_t>(3 * (MOE_E_MAX + 1)); break;
    case MOE_CALL_LAYER: plan_layer(c, s); plan_split(c, s); break;
    case MOE_CALL_LOSS_BACKWARD: plan_loss_backward(c, s); break;
    case MOE_CALL_LAYER_BACKWARD: plan_layer_backward(c, s); break;
    default: return 0;
  }
  return c.used;
}

moe_status moe_route(const moe_shape* s, const void* x, const void* W_r, const float* b,
                     int32_t* topk_idx, float* topk_w, int32_t* n, double* gsum, double* lse2sum,
                     double* hsum, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = moe_check_shape(s);
  if (st != MOE_OK) return st;
  if (expert_choice(s)) return MOE_ERR_UNSUPPORTED;  // runs only through the layer call
  if (!x || !W_r || !topk_idx || !topk_w || !n || !gsum || !lse2sum)
    return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(x) || !aligned16(W_r) || !aligned16(topk_idx) || !aligned16(topk_w))
    return MOE_ERR_INVALID_ARGUMENT;
  if (!ws || ws_bytes < moe_workspace_size(s, MOE_CALL_ROUTE)) return MOE_ERR_WORKSPACE;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  Carve c(ws);
  RoutePlan p = plan_route(c, s);
  hipError_t e = launch_route(s->dtype, s->T, s->d, s->E, s->k, route_flags(s), x, W_r, b, topk_idx,
                              topk_w, p.hist, p.gpart, p.lpart, p.hpart, nullptr, hs);
  if (e != hipSuccess) return MOE_ERR_HIP;
  e = launch_scan(s->T, s->E, -1, static_cast<int>(route_blocks(s)), p.hist, p.gpart, p.lpart,
                  p.hpart, nullptr, n, gsum, lse2sum, hsum, nullptr, nullptr, nullptr, nullptr,
                  gemm_bm(s), hs);
  return hip_status(e);
}

moe_status moe_dispatch(const moe_shape* s, const void* x, const int32_t* topk_idx, void* x_perm,
                        int32_t* perm_token, int32_t* inv_perm, int32_t* offsets, int32_t* counts,
                        int32_t* overflow, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = moe_check_shape(s);
  if (st != MOE_OK) return st;
  if (expert_choice(s)) return MOE_ERR_UNSUPPORTED;  // runs only through the layer call
  if (!topk_idx || !perm_token || !inv_perm || !offsets || !counts || !overflow)
    return MOE_ERR_INVALID_ARGUMENT;
  if (x_perm != nullptr && (!x || !aligned16(x) || !aligned16(x_perm)))
    return MOE_ERR_INVALID_ARGUMENT;
  if (!ws || ws_bytes < moe_workspace_size(s, MOE_CALL_DISPATCH)) return MOE_ERR_WORKSPACE;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  Carve c(ws);
  DispatchPlan p = plan_dispatch(c, s);
  const int64_t C = capacity_of(s);
  hipError_t e = launch_count(s->T, s->E, s->k, topk_idx, p.hist, hs);
  if (e != hipSuccess) return MOE_ERR_HIP;
  e = launch_scan(s->T, s->E, C, static_cast<int>(nblocks(s)), p.hist, nullptr, nullptr, nullptr,
                  p.block_base, counts, nullptr, nullptr, nullptr, nullptr, overflow, offsets,
                  nullptr, gemm_bm(s), hs);
  if (e != hipSuccess) return MOE_ERR_HIP;
  e = launch_scatter(s->T, s->d, s->E, s->k, C, elem_bytes(s), x, topk_idx, kRouteTokens,
                     p.block_base, offsets, x_perm, perm_token, inv_perm, hs);
  return hip_status(e);
}

moe_status moe_expert_ffn(const moe_shape* s, int32_t groups, int32_t Mg, const void* rows,
                          const int32_t* offsets, int64_t max_rows, const void* W_gate,
                          const void* W_up, const void* W_down, void* h, void* out, void* ws,
                          size_t ws_bytes, void* stream) {
  moe_status st = moe_check_shape(s);
  if (st != MOE_OK) return st;
  if (groups < 1 || groups > MOE_E_MAX || Mg < 1 || max_rows < 0 || max_rows > INT32_MAX)
    return groups > MOE_E_MAX ? MOE_ERR_UNSUPPORTED : MOE_ERR_INVALID_ARGUMENT;
  if (Mg % (s->dtype == MOE_F32 ? 4 : 8) != 0) return MOE_ERR_INVALID_ARGUMENT;
  if (Mg > kMaxWidth / 2) return MOE_ERR_UNSUPPORTED;
  if (!rows || !offsets || !W_gate || !W_up || !W_down || !h || !out)
    return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(rows) || !aligned16(W_gate) || !aligned16(W_up) || !aligned16(W_down) ||
      !aligned16(h) || !aligned16(out))
    return MOE_ERR_INVALID_ARGUMENT;
  if (!ws || ws_bytes < moe_workspace_size(s, MOE_CALL_EXPERT_FFN)) return MOE_ERR_WORKSPACE;
  if (max_rows == 0) return MOE_OK;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  int32_t* tile_off = static_cast<int32_t*>(ws);
  const int BM = gemm_bm(s);
  hipError_t e = launch_schedule(groups, offsets, tile_off, BM, hs);
  if (e != hipSuccess) return MOE_ERR_HIP;
  const int64_t max_tiles = cdiv(max_rows, BM) + groups;
  e = launch_gemm_up(s->dtype, groups, s->d, Mg, rows, nullptr, offsets, tile_off, max_tiles,
                     W_gate, W_up, h, hs, max_rows);
  if (e == hipSuccess)
    e = launch_gemm_down(s->dtype, groups, s->d, Mg, offsets, tile_off, max_tiles, W_down, h, out,
                         hs, max_rows);
  return hip_status(e);
}

moe_status moe_combine(const moe_shape* s, const void* out_perm, const int32_t* inv_perm,
                       const float* topk_w, const void* shared_out, void* y, void* stream) {
  moe_status st = moe_check_shape(s);
  if (st != MOE_OK) return st;
  if (expert_choice(s)) return MOE_ERR_UNSUPPORTED;  // runs only through the layer call
  if (!out_perm || !inv_perm || !topk_w || !y) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(out_perm) || !aligned16(y) || (shared_out && !aligned16(shared_out)))
    return MOE_ERR_INVALID_ARGUMENT;
  return hip_status(launch_combine(s->dtype, s->T, s->d, s->k, out_perm, inv_perm, topk_w,
                                   shared_out, y, static_cast<hipStream_t>(stream)));
}

moe_status moe_balance_stats(const moe_shape* s, const int32_t* n, const double* gsum,
                             const double* lse2sum, const double* hsum, float lambda, float* f,
                             float* P, float* aux, float* z, float* diag, const float* b,
                             float* b_new, float gamma, void* stream) {
  moe_status st = moe_check_shape(s);
  if (st != MOE_OK) return st;
  if (!n || !gsum || !lse2sum) return MOE_ERR_INVALID_ARGUMENT;
  if (diag != nullptr && hsum == nullptr) return MOE_ERR_INVALID_ARGUMENT;
  if ((b == nullptr) != (b_new == nullptr)) return MOE_ERR_INVALID_ARGUMENT;
  if (isnan(lambda) || isnan(gamma)) return MOE_ERR_INVALID_ARGUMENT;
  return hip_status(launch_stats(s->T, s->E, stats_fden(s), n, gsum, lse2sum, hsum, lambda, f, P,
                                 aux, z, diag, b, b_new, gamma, static_cast<hipStream_t>(stream)));
}

moe_status moe_layer_forward(const moe_shape* s, const void* x, const void* W_r, const float* b,
                             const void* W_gate, const void* W_up, const void* W_down,
                             const void* Ws_gate, const void* Ws_up, const void* Ws_down, void* y,
                             int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* overflow,
                             float* f, float* P, float* aux, float* z, float* diag, float* b_new,
                             int32_t* inv_perm, int32_t* perm_token, float lambda, float gamma,
                             void* saved, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = moe_check_shape(s);
  if (st != MOE_OK) return st;
  if (!x || !W_r || !W_gate || !W_up || !W_down || !y) return MOE_ERR_INVALID_ARGUMENT;
  if (saved != nullptr && s->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (saved != nullptr && !aligned16(saved)) return MOE_ERR_INVALID_ARGUMENT;
  if (s->S > 0 && (!Ws_gate || !Ws_up || !Ws_down)) return MOE_ERR_INVALID_ARGUMENT;
  if (b_new != nullptr && b == nullptr) return MOE_ERR_INVALID_ARGUMENT;
  // the load-balancing bias is a token-choice device: a per-expert shift cannot change which
  // tokens an expert ranks highest
  if (expert_choice(s) && b != nullptr) return MOE_ERR_INVALID_ARGUMENT;
  if (isnan(lambda) || isnan(gamma)) return MOE_ERR_INVALID_ARGUMENT;
  const void* tensors[] = {x, W_r, W_gate, W_up, W_down, y, topk_idx, topk_w, inv_perm, perm_token};
  for (const void* t : tensors)
    if (t && !aligned16(t)) return MOE_ERR_INVALID_ARGUMENT;
  if (s->S > 0 && (!aligned16(Ws_gate) || !aligned16(Ws_up) || !aligned16(Ws_down)))
    return MOE_ERR_INVALID_ARGUMENT;
  // the workspace must hold plan_layer; the split partials (carved last) are used when it also
  // holds them, as a workspace of moe_workspace_size bytes does
  Carve c0(nullptr);
  plan_layer(c0, s);
  if (!ws || ws_bytes < c0.used) return MOE_ERR_WORKSPACE;

  hipStream_t hs = static_cast<hipStream_t>(stream);
  Carve c(ws);
  LayerPlan p = plan_layer(c, s);
  if (ws_bytes >= moe_workspace_size(s, MOE_CALL_LAYER)) p.part = plan_split(c, s);
  Carve cs(saved);
  const SavedPlan sv = plan_saved(cs, s);  // all NULL when saved is NULL
  int32_t* idx = topk_idx ? topk_idx : p.topk_idx;
  float* w = topk_w ? topk_w : p.topk_w;
  int32_t* n = counts ? counts : p.n;
  int32_t* ovf = overflow ? overflow : p.overflow;
  // placement outputs the caller asked for are written in place of the workspace's copies
  if (inv_perm != nullptr && !expert_choice(s)) p.inv_perm = inv_perm;
  if (perm_token != nullptr) p.perm_token = perm_token;
  const int64_t C = capacity_of(s);
  const int BM = gemm_bm(s);
  const int nblk = static_cast<int>(route_blocks(s));
  const int eb = elem_bytes(s);

  const int64_t max_tiles = cdiv(routed_rows(s), BM) + s->E;

  const bool want_stats = f || P || aux || z || diag || b_new;
  // the shared experts' tile tables come from the selection launch (scan or expert choice)
  int32_t* sh_off = s->S > 0 ? p.sh_offsets : nullptr;
  int32_t* sh_tab = s->S > 0 ? p.sh_tile_off : nullptr;
  StageMarks marks;
  marks.mark(0, hs);
  hipError_t e = hipSuccess;
  if (saved != nullptr && !expert_choice(s))  // the bias this forward selects with, for the backward
    e = launch_copy_f32(b, sv.b, s->E, hs);
  if (e == hipSuccess)
    e = launch_route(s->dtype, s->T, s->d, s->E, s->k, route_flags(s), x, W_r, b, idx, w,
                     p.r.hist, p.r.gpart, p.r.lpart, p.r.hpart, p.cols, hs);
  marks.mark(1, hs);
  if (expert_choice(s)) {
    // every expert's top-r tokens and their tile tables; one more block of the same launch
    // reduces the statistics partials meanwhile
    const RoutePartials rp{p.r.gpart, p.r.lpart, p.r.hpart, nblk, p.gsum, p.lse2sum, p.hsum};
    if (e == hipSuccess)
      e = launch_ec_select(s->T, s->E, static_cast<int>(ec_tokens(s)), p.cols, p.perm_token,
                           p.row_of, p.offsets, n, ovf, p.tile_off, BM, hs, &rp, sh_off, sh_tab);
  } else {
    if (e == hipSuccess)
      e = launch_scan(s->T, s->E, C, nblk, p.r.hist, p.r.gpart, p.r.lpart, p.r.hpart, p.block_base,
                      n, p.gsum, p.lse2sum, p.hsum, p.kept, ovf, p.offsets, p.tile_off, BM, hs,
                      sh_off, sh_tab);
    // placement only: the gate/up GEMM gathers its rows from x through perm_token
    if (e == hipSuccess)
      e = launch_scatter(s->T, s->d, s->E, s->k, C, eb, x, idx, route_block_tokens(s->dtype, s->E, s->T),
                         p.block_base, p.offsets, nullptr, p.perm_token, p.inv_perm, hs);
  }
  marks.mark(2, hs);
  // bf16 inference with shared experts: the shared experts run as a second product of the routed
  // grouped launches (one group of all T rows), so they fill the routed products' last rounds
  const bool fold_shared = s->S > 0 && s->dtype == MOE_BF16 && saved == nullptr;
  const int SM = s->S * s->M;
  const int64_t sh_tiles = cdiv(s->T, BM);
  if (e == hipSuccess && fold_shared) {
    e = launch_gemm_up_shared_bf16(s->E, s->d, s->M, x, p.perm_token, p.offsets, p.tile_off,
                                     max_tiles, W_gate, W_up, p.h, s->T, SM, p.sh_offsets,
                                     p.sh_tile_off, sh_tiles, Ws_gate, Ws_up, p.h_sh, hs);
    marks.mark(3, hs);
    if (e == hipSuccess)
      e = launch_gemm_down_shared_bf16(s->E, s->d, s->M, p.offsets, p.tile_off, max_tiles, W_down,
                                       p.h, p.out_perm, routed_rows(s), s->T, SM, p.sh_offsets,
                                       p.sh_tile_off, sh_tiles, Ws_down, p.h_sh, p.sh, hs, p.part);
    marks.mark(4, hs);
  } else {
    if (e == hipSuccess && saved != nullptr)  // h, and G and U kept for the backward
      e = launch_gemm_up_save_bf16(s->E, s->d, s->M, x, p.perm_token, p.offsets, p.tile_off,
                                   max_tiles, W_gate, W_up, p.h, sv.G, sv.U, hs, s->T);
    else if (e == hipSuccess)
      e = launch_gemm_up(s->dtype, s->E, s->d, s->M, x, p.perm_token, p.offsets, p.tile_off,
                         max_tiles, W_gate, W_up, p.h, hs, s->T);
    marks.mark(3, hs);
    if (e == hipSuccess)
      e = launch_gemm_down(s->dtype, s->E, s->d, s->M, p.offsets, p.tile_off, max_tiles, W_down,
                           p.h, p.out_perm, hs, routed_rows(s), p.part);
    marks.mark(4, hs);
  }
  if (e == hipSuccess && s->S > 0 && !fold_shared) {
    if (saved != nullptr)
      e = launch_gemm_up_save_bf16(1, s->d, SM, x, nullptr, p.sh_offsets, p.sh_tile_off, sh_tiles,
                                   Ws_gate, Ws_up, p.h_sh, sv.Gs, sv.Us, hs, s->T);
    else
      e = launch_gemm_up(s->dtype, 1, s->d, SM, x, nullptr, p.sh_offsets, p.sh_tile_off, sh_tiles,
                         Ws_gate, Ws_up, p.h_sh, hs, s->T);
    if (e == hipSuccess)
      e = launch_gemm_down(s->dtype, 1, s->d, SM, p.sh_offsets, p.sh_tile_off, sh_tiles, Ws_down,
                           p.h_sh, p.sh, hs, s->T);
  }
  marks.mark(5, hs);
  // the combine launch computes the balance statistics in one extra block (the router has read
  // b by now, so b_new may alias it)
  const StatsArgs sa{s->T, s->E, stats_fden(s), n, p.gsum, p.lse2sum, p.hsum, lambda, f, P, aux,
                     z, diag, b_new ? b : nullptr, b_new, gamma};
  const StatsArgs* stats = want_stats ? &sa : nullptr;
  if (e == hipSuccess && expert_choice(s))
    e = launch_combine_ec(s->dtype, s->T, s->d, s->E, s->renorm, p.out_perm, p.row_of,
                          p.cols + static_cast<size_t>(s->E) * s->T, s->S > 0 ? p.sh : nullptr, y,
                          hs, stats);
  else if (e == hipSuccess)
    e = launch_combine(s->dtype, s->T, s->d, s->k, p.out_perm, p.inv_perm, w,
                       s->S > 0 ? p.sh : nullptr, y, hs, stats);
  marks.mark(6, hs);
  marks.mark(7, hs);  // (the statistics stage: inside the combine launch)
  if (e == hipSuccess) e = marks.err;
  return hip_status(e);
}

moe_status moe_layer_forward_noalloc(const moe_shape* s, const void* x, const void* W_r,
                                     const float* b, const void* W_gate, const void* W_up,
                                     const void* W_down, const void* Ws_gate, const void* Ws_up,
                                     const void* Ws_down, void* y, int32_t* topk_idx,
                                     float* topk_w, int32_t* counts, int32_t* overflow, float* f,
                                     float* P, float* aux, float* z, float* diag, float* b_new,
                                     int32_t* inv_perm, int32_t* perm_token, float lambda,
                                     float gamma, void* saved, void* stream) {
  moe_status st = moe_check_shape(s);
  if (st != MOE_OK) return st;
  // the scratch must hold the layer's plan; the split partials are used when they fit as well
  Carve c0(nullptr);
  plan_layer(c0, s);
  if (c0.used > MOE_SCRATCH_BYTES) return MOE_ERR_SCRATCH;
  // every argument check of the allocating call, before the scratch is looked up: a dry run with
  // a null workspace fails only on the workspace if everything else is valid
  st = moe_layer_forward(s, x, W_r, b, W_gate, W_up, W_down, Ws_gate, Ws_up, Ws_down, y, topk_idx,
                         topk_w, counts, overflow, f, P, aux, z, diag, b_new, inv_perm,
                         perm_token, lambda, gamma, saved, nullptr, 0, stream);
  if (st != MOE_ERR_WORKSPACE) return st == MOE_OK ? MOE_ERR_HIP : st;
  void* ws = nullptr;
  st = current_scratch(&ws);
  if (st != MOE_OK) return st;
  return moe_layer_forward(s, x, W_r, b, W_gate, W_up, W_down, Ws_gate, Ws_up, Ws_down, y,
                           topk_idx, topk_w, counts, overflow, f, P, aux, z, diag, b_new, inv_perm,
                           perm_token, lambda, gamma, saved, ws, MOE_SCRATCH_BYTES, stream);
}

moe_status moe_balance_loss_backward(const moe_shape* s, const void* x, const void* W_r,
                                     const int32_t* n, float lambda, float z_coef,
                                     float* dlogits, float* dW_r, float* dx, void* ws,
                                     size_t ws_bytes, void* stream) {
  moe_status st = moe_check_shape(s);
  if (st != MOE_OK) return st;
  if (!x || !W_r || !n || (!dlogits && !dW_r && !dx)) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(x) || !aligned16(W_r)) return MOE_ERR_INVALID_ARGUMENT;
  if (isnan(lambda) || isnan(z_coef)) return MOE_ERR_INVALID_ARGUMENT;
  if (s->T * static_cast<int64_t>(s->E) > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < moe_workspace_size(s, MOE_CALL_LOSS_BACKWARD)) return MOE_ERR_WORKSPACE;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  Carve c(ws);
  LossBackwardPlan p = plan_loss_backward(c, s);
  const size_t ET = static_cast<size_t>(s->E) * s->T;
  // the router in its column mode recomputes the logits and scores
  hipError_t e = launch_route(s->dtype, s->T, s->d, s->E, s->k, route_flags(s) | kRouteExpertChoice,
                              x, W_r, nullptr, nullptr, nullptr, p.r.hist, p.r.gpart, p.r.lpart,
                              p.r.hpart, p.cols, hs);
  if (e == hipSuccess)
    e = launch_loss_grad(s->T, s->E, s->scoring == MOE_SCORE_SIGMOID, p.cols, p.cols + ET, n,
                         stats_fden(s), lambda, z_coef, dlogits ? dlogits : p.dl, p.dlT, hs);
  if (e == hipSuccess && dW_r)  // dW_r [E][d] = sum_t dl[t][e] x[t][:], over token ranges
    e = launch_kmajor_gemm(s->dtype, s->E, s->d, s->T, p.ks_w, dlogits ? dlogits : p.dl, x, dW_r,
                           p.partial, hs);
  if (e == hipSuccess && dx)  // dx [T][d] = sum_e dl[e][t] W_r[e][:]
    e = launch_kmajor_gemm(s->dtype, s->T, s->d, s->E, 1, p.dlT, W_r, dx, nullptr, hs);
  return hip_status(e);
}

moe_status moe_layer_backward(const moe_shape* s, const void* x, const void* W_r, const float* b,
                              const void* W_gate, const void* W_up, const void* W_down,
                              const void* Ws_gate, const void* Ws_up, const void* Ws_down,
                              const void* dy, float lambda, float z_coef, float* dx, float* dW_r,
                              float* dW_gate, float* dW_up, float* dW_down, float* dWs_gate,
                              float* dWs_up, float* dWs_down, int32_t* topk_idx,
                              const void* saved, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = moe_check_shape(s);
  if (st != MOE_OK) return st;
  if (expert_choice(s) && b != nullptr) return MOE_ERR_INVALID_ARGUMENT;
  if (saved != nullptr && s->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (saved != nullptr && !aligned16(saved)) return MOE_ERR_INVALID_ARGUMENT;
  if (!x || !W_r || !W_gate || !W_up || !W_down || !dy) return MOE_ERR_INVALID_ARGUMENT;
  if (!dx || !dW_r || !dW_gate || !dW_up || !dW_down) return MOE_ERR_INVALID_ARGUMENT;
  if (s->S > 0 && (!Ws_gate || !Ws_up || !Ws_down || !dWs_gate || !dWs_up || !dWs_down))
    return MOE_ERR_INVALID_ARGUMENT;
  if (isnan(lambda) || isnan(z_coef)) return MOE_ERR_INVALID_ARGUMENT;
  if (s->T * static_cast<int64_t>(s->E) > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  // bf16 layers read an expert's [W_gate; W_up] (and the shared experts') in place, with 32-bit
  // byte offsets inside it
  const int64_t gu_bytes = static_cast<int64_t>(s->M) * s->d * 4;
  if (s->dtype == MOE_BF16 && (gu_bytes >= (int64_t{1} << 32) || s->S * gu_bytes >= (int64_t{1} << 32)))
    return MOE_ERR_UNSUPPORTED;
  const void* tensors[] = {x, W_r, W_gate, W_up, W_down, dy};
  for (const void* t : tensors)
    if (!aligned16(t)) return MOE_ERR_INVALID_ARGUMENT;
  if (s->S > 0 && (!aligned16(Ws_gate) || !aligned16(Ws_up) || !aligned16(Ws_down)))
    return MOE_ERR_INVALID_ARGUMENT;
  if (!ws || ws_bytes < moe_workspace_size(s, MOE_CALL_LAYER_BACKWARD)) return MOE_ERR_WORKSPACE;

  hipStream_t hs = static_cast<hipStream_t>(stream);
  Carve c(ws);
  LayerBackwardPlan p = plan_layer_backward(c, s);
  LayerPlan& f = p.f;
  const float* b_sel = b;  // the bias the selection is made with
  if (saved != nullptr) {  // the forward's pre-activations replace the recomputed ones
    Carve cs(const_cast<void*>(saved));  // read only
    const SavedPlan sv = plan_saved(cs, s);
    p.G = sv.G;
    p.U = sv.U;
    p.Gs = sv.Gs;
    p.Us = sv.Us;
    if (!expert_choice(s)) b_sel = sv.b;  // as the forward selected, whatever b holds now
  }
  int32_t* idx = topk_idx ? topk_idx : f.topk_idx;
  const int64_t C = capacity_of(s);
  const int BM = gemm_bm(s);
  const int nblk = static_cast<int>(route_blocks(s));
  const int eb = elem_bytes(s);
  const int64_t R = routed_rows(s);
  const int64_t max_tiles = cdiv(R, BM) + s->E;
  const int64_t max_t64 = cdiv(R, 64) + s->E;
  const int64_t dM = static_cast<int64_t>(s->d) * s->M;
  const size_t ET = static_cast<size_t>(s->E) * s->T;
  // ---- forward recompute: routing, placement, fp32 pre-activations and h, score columns
  const bool ec = expert_choice(s);
  const float* lcol = p.cols;
  const float* scol = p.cols + ET;
  hipError_t e = hipSuccess;
  if (ec) {  // logit and score columns, then every expert's top-r tokens and the tile tables
    e = launch_route(s->dtype, s->T, s->d, s->E, s->k, route_flags(s), x, W_r, nullptr, nullptr,
                     nullptr, f.r.hist, f.r.gpart, f.r.lpart, f.r.hpart, p.cols, hs);
    if (e == hipSuccess)
      e = launch_ec_select(s->T, s->E, static_cast<int>(ec_tokens(s)), lcol, f.perm_token,
                           f.row_of, f.offsets, f.n, f.overflow, f.tile_off, BM, hs);
  } else {
    e = launch_route(s->dtype, s->T, s->d, s->E, s->k, route_flags(s), x, W_r, b_sel, idx,
                     f.topk_w, f.r.hist, f.r.gpart, f.r.lpart, f.r.hpart, nullptr, hs);
    if (e == hipSuccess)
      e = launch_scan(s->T, s->E, C, nblk, f.r.hist, nullptr, nullptr, nullptr, f.block_base, f.n,
                      nullptr, nullptr, nullptr, f.kept, f.overflow, f.offsets, f.tile_off, BM, hs);
    if (e == hipSuccess)
      e = launch_scatter(s->T, s->d, s->E, s->k, C, eb, x, idx,
                         route_block_tokens(s->dtype, s->E, s->T), f.block_base, f.offsets, nullptr,
                         f.perm_token, f.inv_perm, hs);
  }
  if (s->dtype == MOE_BF16) {  // G and U in one launch (gate and up tiles paired), unless kept
    if (e == hipSuccess && saved == nullptr)
      e = launch_gemm_gu_f32out_bf16(s->E, s->d, s->M, x, f.perm_token, f.offsets, f.tile_off,
                                     max_tiles, W_gate, W_up, p.G, p.U, hs, s->T);
  } else {
    if (e == hipSuccess)
      e = launch_gemm_plain(s->dtype, s->E, x, f.perm_token, f.offsets, f.tile_off, max_tiles,
                            W_gate, dM, s->M, s->d, p.G, hs);
    if (e == hipSuccess)
      e = launch_gemm_plain(s->dtype, s->E, x, f.perm_token, f.offsets, f.tile_off, max_tiles,
                            W_up, dM, s->M, s->d, p.U, hs);
    if (e == hipSuccess) e = launch_swiglu_fwd(R * s->M, p.G, p.U, p.h, hs);
  }
  if (e == hipSuccess && !ec)
    e = launch_route(s->dtype, s->T, s->d, s->E, s->k, route_flags(s) | kRouteExpertChoice, x, W_r,
                     nullptr, nullptr, nullptr, f.r.hist, f.r.gpart, f.r.lpart, f.r.hpart, p.cols,
                     hs);
  // 64-row tiles; on MFMA the weight-gradient column ranges, at least two k-slices per expert
  const bool mfma = s->dtype == MOE_BF16;
  if (e == hipSuccess) e = launch_schedule(s->E, f.offsets, p.tile64, 64, hs, mfma ? 2 : 0);
  const int d = s->d, M = s->M;
  // ---- combine: P_row = dy_t W_down[e] gives d w = <P, h> and dh = w P, hence dG, dU
  if (e == hipSuccess && mfma)  // W_down[e] read in place as the [d][M] B operand
    e = launch_gemm_kn_bf16(s->E, dy, f.perm_token, f.offsets, f.tile_off, max_tiles, W_down,
                            nullptr, dM, M, d, p.P, hs);
  else if (e == hipSuccess)
    e = launch_nn_gemm(s->dtype, s->dtype, false, dy, nullptr, f.perm_token, f.offsets, p.tile64,
                       s->E, max_t64, W_down, nullptr, dM, s->M, s->d, p.P, hs);
  if (e == hipSuccess && ec)  // expert choice: the gate of every row first
    e = launch_ec_gates(s->T, s->E, s->renorm, f.row_of, scol, p.wrow, hs);
  if (e == hipSuccess)
    e = launch_bw_rows(s->dtype, f.offsets, s->E, R, s->d, s->M, s->k, f.perm_token,
                       ec ? nullptr : f.inv_perm, f.topk_w, dy, p.P, p.G, p.U, p.dw, p.dG, p.dU,
                       p.dGU, p.wh, p.dout, p.wrow, hs);
  const int sig = s->scoring == MOE_SCORE_SIGMOID;
  if (e == hipSuccess && ec)
    e = launch_bw_router_ec(s->T, s->E, s->renorm, sig, f.row_of, lcol, scol, p.dw, f.n,
                            stats_fden(s), lambda, z_coef, p.dl, p.dlT, hs);
  else if (e == hipSuccess)
    e = launch_bw_router(s->T, s->E, s->k, s->renorm, sig, lcol, scol, idx, f.inv_perm, f.topk_w,
                         p.dw, f.n, stats_fden(s), lambda, z_coef, p.dl, p.dlT, hs);
  // ---- routed experts
  if (mfma) {
    if (e == hipSuccess)  // dx_row = [dG dU] [W_gate[e]; W_up[e]] over K = 2M, weights in place
      e = launch_gemm_kn_bf16(s->E, p.dGU, nullptr, f.offsets, f.tile_off, max_tiles, W_gate,
                              W_up, dM, d, 2 * M, p.dxr, hs, p.part_dx);
    // the weight gradients read their row operands in place, K-major: w h (written by bw_rows),
    // [dG | dU], and the dy and x rows of the kept rows, gathered into routed order
    const bf16_t* dGU = static_cast<const bf16_t*>(p.dGU);
    if (e == hipSuccess) e = launch_gather_rows(dy, d, f.perm_token, f.offsets, s->E, R, p.dyr, hs);
    if (e == hipSuccess) e = launch_gather_rows(x, d, f.perm_token, f.offsets, s->E, R, p.xr, hs);
    if (e == hipSuccess)  // dW_down[e] = sum over its rows of dy_t^T (w h)
      e = launch_gemm_wgrad_bf16(p.dyr, d, p.wh, M, R, f.offsets, p.tile64, s->E, d, M, dW_down,
                                 hs);
    if (e == hipSuccess)  // dW_gate[e] = dG_e^T x_e
      e = launch_gemm_wgrad_bf16(dGU, 2 * M, p.xr, d, R, f.offsets, p.tile64, s->E, M, d, dW_gate,
                                 hs);
    if (e == hipSuccess)
      e = launch_gemm_wgrad_bf16(dGU + M, 2 * M, p.xr, d, R, f.offsets, p.tile64, s->E, M, d,
                                 dW_up, hs);
  }
  if (e == hipSuccess && !mfma)  // dx_row = dG W_gate[e] + dU W_up[e]
    e = launch_nn_gemm(MOE_F32, s->dtype, true, p.dG, p.dU, nullptr, f.offsets, p.tile64, s->E,
                       max_t64, W_gate, W_up, dM, s->d, s->M, p.dxr, hs);
  if (e == hipSuccess && !mfma)  // dW_down[e] = sum_rows d out^T h
    e = launch_kk_gemm(MOE_F32, MOE_F32, p.dout, s->d, p.h, s->M, nullptr, f.offsets, s->E,
                       dW_down, hs);
  if (e == hipSuccess && !mfma)  // dW_gate[e] = sum_rows dG^T x
    e = launch_kk_gemm(MOE_F32, s->dtype, p.dG, s->M, x, s->d, f.perm_token, f.offsets, s->E,
                       dW_gate, hs);
  if (e == hipSuccess && !mfma)
    e = launch_kk_gemm(MOE_F32, s->dtype, p.dU, s->M, x, s->d, f.perm_token, f.offsets, s->E,
                       dW_up, hs);
  // ---- router weights and the router part of dx
  if (e == hipSuccess)
    e = launch_kmajor_gemm(s->dtype, s->E, s->d, s->T, p.ks_w, p.dl, x, dW_r, p.partial, hs);
  if (e == hipSuccess)
    e = launch_kmajor_gemm(s->dtype, s->T, s->d, s->E, 1, p.dlT, W_r, dx, nullptr, hs);
  // ---- shared experts: one group of all T rows, output gradient dy
  if (e == hipSuccess && s->S > 0) {
    const int SM = s->S * s->M;
    const int64_t sh_tiles = cdiv(s->T, BM);
    const int64_t dSM = static_cast<int64_t>(s->d) * SM;
    e = launch_shared_table(s->T, BM, f.sh_offsets, f.sh_tile_off, hs);
    if (mfma) {
      if (e == hipSuccess && saved == nullptr)
        e = launch_gemm_gu_f32out_bf16(1, s->d, SM, x, nullptr, f.sh_offsets, f.sh_tile_off,
                                       sh_tiles, Ws_gate, Ws_up, p.Gs, p.Us, hs, s->T);
    } else {
      if (e == hipSuccess)
        e = launch_gemm_plain(s->dtype, 1, x, nullptr, f.sh_offsets, f.sh_tile_off, sh_tiles,
                              Ws_gate, dSM, SM, s->d, p.Gs, hs);
      if (e == hipSuccess)
        e = launch_gemm_plain(s->dtype, 1, x, nullptr, f.sh_offsets, f.sh_tile_off, sh_tiles,
                              Ws_up, dSM, SM, s->d, p.Us, hs);
      if (e == hipSuccess)
        e = launch_swiglu_fwd(static_cast<int64_t>(s->T) * SM, p.Gs, p.Us, p.hs, hs);
    }
    if (e == hipSuccess) e = launch_schedule(1, f.sh_offsets, p.sh_tile64, 64, hs, mfma ? 2 : 0);
    const int64_t sh_t64 = cdiv(s->T, 64) + 1;
    if (mfma) {
      const bf16_t* dGUs = static_cast<const bf16_t*>(p.dGUs);
      if (e == hipSuccess)  // dhs = dy Ws_down (Ws_down [d][SM] read in place)
        e = launch_gemm_kn_bf16(1, dy, nullptr, f.sh_offsets, f.sh_tile_off, sh_tiles, Ws_down,
                                nullptr, 0, SM, d, p.dhs, hs);
      if (e == hipSuccess)
        e = launch_swiglu_bw_cat(s->T, SM, p.dhs, p.Gs, p.Us, p.dGUs, p.hsb, hs);
      if (e == hipSuccess)  // dxs = [dGs dUs] [Ws_gate; Ws_up] over K = 2 SM
        e = launch_gemm_kn_bf16(1, p.dGUs, nullptr, f.sh_offsets, f.sh_tile_off, sh_tiles, Ws_gate,
                                Ws_up, 0, d, 2 * SM, p.dxs, hs);
      // the weight gradients over all T rows, read in place: dy, h, [dGs | dUs] and x; over
      // ks_sh row ranges when one range's tiles would leave most compute units idle, each range
      // a group of the persistent product writing its own partial, summed in range order
      const int ks = p.ks_sh;
      const int32_t* so = ks > 1 ? p.sh_split_off : f.sh_offsets;
      const int32_t* skt = ks > 1 ? p.sh_split_kt : p.sh_tile64;
      if (e == hipSuccess && ks > 1) e = launch_row_splits(s->T, ks, p.sh_split_off, hs);
      if (e == hipSuccess && ks > 1) e = launch_schedule(ks, p.sh_split_off, p.sh_split_kt, 64, hs, 2);
      auto sh_wgrad = [&](const void* A, int lda, const void* B, int ldb, int Ma, int Nb,
                          float* out) {
        hipError_t r = launch_gemm_wgrad_bf16(A, lda, B, ldb, s->T, so, skt, ks, Ma, Nb,
                                              ks > 1 ? p.sh_wpart : out, hs);
        if (r == hipSuccess && ks > 1)
          r = launch_sum_ranges(static_cast<int64_t>(Ma) * Nb, ks, p.sh_wpart, out, hs);
        return r;
      };
      if (e == hipSuccess) e = sh_wgrad(dy, d, p.hsb, SM, d, SM, dWs_down);
      if (e == hipSuccess) e = sh_wgrad(dGUs, 2 * SM, x, d, SM, d, dWs_gate);
      if (e == hipSuccess) e = sh_wgrad(dGUs + SM, 2 * SM, x, d, SM, d, dWs_up);
    } else {
      if (e == hipSuccess)
        e = launch_nn_gemm(s->dtype, s->dtype, false, dy, nullptr, nullptr, f.sh_offsets,
                           p.sh_tile64, 1, sh_t64, Ws_down, nullptr, dSM, SM, s->d, p.dhs, hs);
      if (e == hipSuccess)
        e = launch_swiglu_bw(MOE_F32, static_cast<int64_t>(s->T) * SM, p.dhs, p.Gs, p.Us, p.dGs,
                             p.dUs, hs);
      if (e == hipSuccess)
        e = launch_nn_gemm(MOE_F32, s->dtype, true, p.dGs, p.dUs, nullptr, f.sh_offsets,
                           p.sh_tile64, 1, sh_t64, Ws_gate, Ws_up, dSM, s->d, SM, p.dxs, hs);
      if (e == hipSuccess)
        e = launch_kk_gemm(s->dtype, MOE_F32, dy, s->d, p.hs, SM, nullptr, f.sh_offsets, 1,
                           dWs_down, hs);
      if (e == hipSuccess)
        e = launch_kk_gemm(MOE_F32, s->dtype, p.dGs, SM, x, s->d, nullptr, f.sh_offsets, 1,
                           dWs_gate, hs);
      if (e == hipSuccess)
        e = launch_kk_gemm(MOE_F32, s->dtype, p.dUs, SM, x, s->d, nullptr, f.sh_offsets, 1, dWs_up,
                           hs);
    }
  }
  // ---- tokens
  if (e == hipSuccess && ec)
    e = launch_bw_dx_ec(s->T, s->d, s->E, f.row_of, p.dxr, s->S > 0 ? p.dxs : nullptr, dx, hs);
  else if (e == hipSuccess)
    e = launch_bw_dx(s->T, s->d, s->k, f.inv_perm, p.dxr, s->S > 0 ? p.dxs : nullptr, dx, hs);
  return hip_status(e);
}

moe_status moe_set_stage_events(void* const* events, int count) {
  std::lock_guard<std::mutex> lock(g_stage_mu);
  if (events == nullptr) {
    g_stage_on = false;
    for (int i = 0; i < MOE_STAGE_COUNT; ++i) g_stage_events[i] = nullptr;
    return MOE_OK;
  }
  if (count < MOE_STAGE_COUNT) return MOE_ERR_INVALID_ARGUMENT;
  for (int i = 0; i < MOE_STAGE_COUNT; ++i) g_stage_events[i] = static_cast<hipEvent_t>(events[i]);
  g_stage_on = true;
  return MOE_OK;
}

}  // extern "C"

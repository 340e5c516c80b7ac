/*
 * moe.h -- C ABI of the MI355X (gfx950) sparse Mixture-of-Experts FFN layer forward.
 *
 * The layer computes, for every token x_t of a routing batch of T tokens,
 *
 *     y_t = sum_{e in S_t} w_te * E_e(x_t)  +  sum_{s < S} E^s(x_t)
 *
 * with router probabilities g_t = softmax(W_r x_t) (or per-expert sigmoid scores, the DeepSeek-V3
 * gate), selection S_t = TopK(g_t + b) over the routed experts, gates w_te = g_te renormalised
 * over S_t, SwiGLU experts
 * E_e(x) = W_down,e (SiLU(W_gate,e x) ⊙ (W_up,e x)), optional shared experts applied to every
 * token, and an optional per-expert capacity C = ceil(c k T / E) that drops overflow assignments.
 * Alongside it come the balance statistics f_e, P_e, aux = lambda E sum_e f_e P_e and the router
 * z-loss. Sources (page title, section):
 *   - "MoE：条件计算与路由": core formula; §原理与演进 (g = softmax(W_r x), TopK, L_balance);
 *     §无辅助损失负载均衡（ALF-LB） (bias b_e before Top-K, rule-based update); §1 (loads n_e);
 *     §3 (C = ceil(c B k / E), token dropping); §7 eqs. (1)-(3) (renormalised gates, y).
 *   - "深入理解 MoE (混合专家模型)：稀疏激活与高效扩展": §4.2.1 (f_i, P_i, alpha = 0.01);
 *     §10.2 / §11 (SwiGLU(x) = SiLU(W_1 x) ⊙ (W_3 x), W_2 projects back).
 *   - "MOE大模型对比篇": §2.1 (balance loss), §2.2 (z-loss), §3.3 (shared experts).
 *   - the adg.csdn.net MoE notes page: §九 (DeepSeek-V3 scores experts with a sigmoid).
 *
 * Conventions for every entry point:
 *   - Pointers named as device buffers are device pointers owned by the caller; tensors are dense,
 *     row-major and 16-byte aligned. The library never allocates, frees or keeps a pointer past
 *     the call. Scratch memory is the caller's workspace, sized by moe_workspace_size().
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and is complete when
 *     the caller synchronises that stream. No entry point synchronises.
 *   - All argument checks run on the host before anything is enqueued: on an error the call
 *     returns a status and enqueues nothing. A failed kernel launch returns MOE_ERR_HIP;
 *     asynchronous faults surface at the caller's synchronisation.
 *   - Results are deterministic: the same inputs give bit-identical outputs on every call.
 *   - Entry points are stateless and re-entrant; concurrent calls must use distinct workspaces.
 *     The one exception is the profiling hook moe_set_stage_events (process-wide, under a lock).
 *   - dtype MOE_BF16: x, weights, intermediates and y are bf16, products accumulate in fp32, the
 *     routing arithmetic is fp32, h and expert outputs are rounded to bf16, y is rounded once.
 *     dtype MOE_F32: all of these are fp32.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1, /* a size, pointer, alignment or flag is invalid            */
  MOE_ERR_UNSUPPORTED = 2,      /* valid, but beyond this build's limits (E, k, dtype)       */
  MOE_ERR_WORKSPACE = 3,        /* workspace missing or smaller than moe_workspace_size()    */
  MOE_ERR_HIP = 4,              /* a kernel launch failed                                   */
  MOE_ERR_SCRATCH = 5           /* moe_layer_forward_noalloc: the shape needs more workspace
                                   than its static scratch (MOE_SCRATCH_BYTES)               */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Who chooses: every token its top-k experts, or every expert its top-r tokens. */
typedef enum {
  MOE_ROUTE_TOKEN_CHOICE = 0,  /* S_t = TopK_e(g_t + b), capacity C drops the overflow         */
  MOE_ROUTE_EXPERT_CHOICE = 1  /* expert e takes the r = min(C, T) tokens of largest l_te      */
} moe_routing;

/* How the router scores the experts from the logits l_te. */
typedef enum {
  MOE_SCORE_SOFTMAX = 0, /* g_te = softmax_e(l_t)                                        */
  MOE_SCORE_SIGMOID = 1  /* g_te = 1 / (1 + exp(-l_te)), each expert on its own          */
} moe_scoring;

/* Which entry point a workspace is sized for. */
typedef enum {
  MOE_CALL_ROUTE = 0,
  MOE_CALL_DISPATCH = 1,
  MOE_CALL_EXPERT_FFN = 2,
  MOE_CALL_LAYER = 3,
  MOE_CALL_LOSS_BACKWARD = 4,
  MOE_CALL_LAYER_BACKWARD = 5
} moe_call;

#define MOE_E_MAX 256 /* routed experts per layer */
#define MOE_K_MAX 16  /* experts chosen per token */

/* Layer sizes, in the pages' notation. */
typedef struct {
  int64_t T;      /* tokens in the routing batch (B on the pages), >= 1                       */
  int32_t d;      /* hidden size; multiple of 8 (bf16) or 4 (fp32); at most 2^21              */
  int32_t E;      /* routed experts, 1 <= E <= MOE_E_MAX                                      */
  int32_t k;      /* experts chosen per token, 1 <= k <= min(E, MOE_K_MAX)                    */
  int32_t M;      /* expert intermediate width; multiple of 8 (bf16) or 4 (fp32); at most 2^20 */
  int32_t S;      /* shared experts, each of width M, >= 0; they run as one expert of width S*M
                     (S*M at most 2^20)                                                        */
  float c;        /* capacity factor; <= 0 means no capacity limit; NaN is invalid            */
  int32_t renorm; /* 1: renormalise the chosen gates over S_t; 0: use g_te as is               */
  int32_t dtype;  /* moe_dtype                                                                */
  int32_t scoring; /* moe_scoring                                                             */
  int32_t routing; /* moe_routing; expert choice runs only through moe_layer_forward          */
} moe_shape;

/* Short text for a status code (static storage). */
const char* moe_status_string(int status);

/* Checks a shape as the entry points do; MOE_OK if every entry point accepts it. */
moe_status moe_check_shape(const moe_shape* s);

/* Capacity C = ceil(c k T / E) of "MoE：条件计算与路由" §3, computed in double precision as
 * ((c * k) * T) / E from the float c; -1 when c <= 0 (no limit) or the shape is invalid. */
int64_t moe_capacity(const moe_shape* s);

/* Bytes of workspace entry point `call` needs for shape s (0 if the shape is invalid).
 * For MOE_CALL_EXPERT_FFN the size is for groups = E (it also covers groups = 1). */
size_t moe_workspace_size(const moe_shape* s, int call);

/* Rows R of the layer's expert-contiguous routed buffers: min(T k, E C) for token choice (T k
 * without a capacity), E r for expert choice; -1 if the shape is invalid. perm_token of
 * moe_layer_forward holds R entries. */
int64_t moe_routed_rows(const moe_shape* s);

/*
 * moe_saved_size -- bytes of the buffer in which moe_layer_forward keeps, for a later
 * moe_layer_backward on the same inputs, the fp32 gate and up pre-activations of every routed row
 * and of the shared experts (bf16 layers only; 0 for fp32 layers or an invalid shape). Layout
 * (256-byte aligned parts): G, U [R, M] each, R = moe_routed_rows(s) rows in the forward's
 * expert-major row order, then Gs, Us [T, S*M] each when S > 0, then the bias the forward
 * selected with, [E] fp32 (zeros when it had none; token choice only).
 */
size_t moe_saved_size(const moe_shape* s);

/*
 * moe_route -- router of "MoE：条件计算与路由" §原理与演进 and §无辅助损失负载均衡（ALF-LB）.
 *
 * For every token t: l_te = sum_i x_ti W_r,ei (no router bias); m = max_e l_te,
 * lse_t = m + ln sum_e exp(l_te - m), g_te = exp(l_te - lse_t) (MOE_SCORE_SOFTMAX) or
 * g_te = 1 / (1 + exp(-l_te)) (MOE_SCORE_SIGMOID); s_te = g_te + b_e (b optional);
 * S_t = the k experts of largest s_te, in descending s order, equal scores to the lower index;
 * w_tj = g_t,S_tj / sum_j' g_t,S_tj' (or g_t,S_tj when renorm == 0).
 *   x        device [T, d] (dtype)          W_r   device [E, d] (dtype)
 *   b        device [E] fp32 or NULL (selection only; gates use the unbiased g)
 *   topk_idx device out [T, k] int32        topk_w device out [T, k] fp32
 *   n        device out [E] int32: loads n_e = #{t : e in S_t}, before any capacity limit
 *   gsum     device out [E] double: sum_t p_te, p = g (softmax) or g_te / sum_e' g_te' (sigmoid)
 *   lse2sum  device out [1] double: sum_t lse_t^2 (raw logits, either scoring)
 *   hsum     device out [1] double or NULL: sum_t H(p_t), H(p) = -sum_e p_e ln p_e, the routing
 *            entropy of "MoE：条件计算与路由" §9
 *   ws       device workspace of moe_workspace_size(s, MOE_CALL_ROUTE) bytes
 */
moe_status moe_route(const moe_shape* s, const void* x, const void* W_r, const float* b,
                     int32_t* topk_idx, float* topk_w, int32_t* n, double* gsum, double* lse2sum,
                     double* hsum, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_dispatch -- capacity and expert-contiguous placement ("MoE：条件计算与路由" §3; the
 * per-expert histogram, sort and gather of the DeepseekV3MoE listing on the adg.csdn.net notes
 * page, §四).
 *
 * Position p(t, e) = number of tokens t' < t with e in S_t'. The assignment (t, j), e = S_tj, is
 * kept iff C < 0 or p < C; kept_e = min(n_e, C); overflow_e = n_e - kept_e;
 * offsets_e = sum_{e' < e} kept_e'; its row is offsets_e + p. Rows of one expert are therefore in
 * ascending token order.
 *   x          device [T, d] (dtype)
 *   topk_idx   device [T, k] int32, each row k distinct experts in [0, E)
 *   x_perm     device out [T*k, d] (dtype) or NULL (row copy skipped): x_perm[row] = x[t]
 *   perm_token device out [T*k] int32: perm_token[row] = t for rows < offsets[E]; others unset
 *   inv_perm   device out [T, k] int32: row of (t, j), or -1 if dropped
 *   offsets    device out [E+1] int32    counts device out [E] int32 (n_e)
 *   overflow   device out [E] int32 (dropped assignments per expert)
 *   ws         device workspace of moe_workspace_size(s, MOE_CALL_DISPATCH) bytes
 * Out-of-range expert ids in topk_idx are a caller error (not detected).
 */
moe_status moe_dispatch(const moe_shape* s, const void* x, const int32_t* topk_idx, void* x_perm,
                        int32_t* perm_token, int32_t* inv_perm, int32_t* offsets, int32_t* counts,
                        int32_t* overflow, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_expert_ffn -- grouped SwiGLU experts ("深入理解 MoE ..." §10.2: SiLU(W_1 x) ⊙ (W_3 x),
 * then W_2; no biases). Group g owns rows [offsets_g, offsets_{g+1}) of `rows` and weights
 * W_gate[g], W_up[g] ([Mg, d] each) and W_down[g] ([d, Mg]):
 *     h[r]   = SiLU(rows[r] W_gate[g]^T) ⊙ (rows[r] W_up[g]^T)      (rounded to dtype)
 *     out[r] = h[r] W_down[g]^T                                     (rounded to dtype)
 * Shared experts use groups = 1, offsets = {0, T}, rows = x and Mg = S*M.
 *   groups   1 <= groups <= MOE_E_MAX      Mg  intermediate width of every group (mult. of 8/4)
 *   rows     device [max_rows, d]          offsets device [groups+1] int32, non-decreasing,
 *                                          offsets[0] = 0, offsets[groups] <= max_rows
 *   W_gate, W_up device [groups, Mg, d]    W_down device [groups, d, Mg]
 *   h        device out [max_rows, Mg]     out device out [max_rows, d]; rows >= offsets[groups]
 *                                          are left untouched
 *   ws       device workspace of moe_workspace_size(s, MOE_CALL_EXPERT_FFN) bytes
 * The hidden size d and dtype come from s; s->M and s->E are not used.
 */
moe_status moe_expert_ffn(const moe_shape* s, int32_t groups, int32_t Mg, const void* rows,
                          const int32_t* offsets, int64_t max_rows, const void* W_gate,
                          const void* W_up, const void* W_down, void* h, void* out, void* ws,
                          size_t ws_bytes, void* stream);

/*
 * moe_combine -- gate-weighted un-permute and sum ("MoE：条件计算与路由" §7 eq. (3)):
 *     y_t = sum_{j : inv_perm_tj >= 0} w_tj * out_perm[inv_perm_tj]  (+ shared_out_t)
 * summed in fp32 in slot order j = 0..k-1, then the shared term, rounded once to dtype.
 *   out_perm   device [rows, d] (dtype)    inv_perm device [T, k] int32 (-1 = dropped)
 *   topk_w     device [T, k] fp32          shared_out device [T, d] (dtype) or NULL
 *   y          device out [T, d] (dtype)
 */
moe_status moe_combine(const moe_shape* s, const void* out_perm, const int32_t* inv_perm,
                       const float* topk_w, const void* shared_out, void* y, void* stream);

/*
 * moe_balance_stats -- balance statistics and the loss-free-balancing bias step.
 *   f_e = n_e / (k T)   P_e = gsum_e / T   aux = lambda E sum_e f_e P_e
 *   ("MoE：条件计算与路由" §原理与演进; "深入理解 MoE ..." §4.2.1; "MOE大模型对比篇" §2.1)
 *   z = lse2sum / T   ("MOE大模型对比篇" §2.2 z-loss, natural log, raw router logits)
 *   b_new_e = b_e + gamma * sign(k T / E - n_e) in fp32, sign(0) = 0 ("MoE：条件计算与路由"
 *   §无辅助损失负载均衡（ALF-LB）: overloaded experts' bias goes down, underloaded up)
 * f_e uses k T so that sum_e f_e = 1 for any k (the argmax fraction when k = 1).
 * Routing diagnostics (diag, nullable; "MoE：条件计算与路由" §9-§10; importance CV^2 of the
 * adg.csdn.net notes page): diag[0] = hsum / T (mean routing entropy, natural log),
 *   diag[1] = sum_ij |n_i - n_j| / (2 E sum_e n_e) (load Gini coefficient),
 *   diag[2] = max_e n_e / mean_e n_e, diag[3] = Var_e(gsum) / Mean_e(gsum)^2 (population).
 *   n [E] int32, gsum [E] double, lse2sum [1] double, hsum [1] double: device, as written by
 *   moe_route (hsum may be NULL when diag is NULL)
 *   f, P device out [E] fp32 (nullable)    aux, z device out [1] fp32 (nullable)
 *   diag device out [4] fp32 (nullable)
 *   b device [E] fp32 and b_new device out [E] fp32: both NULL, or both set (may alias)
 */
moe_status moe_balance_stats(const moe_shape* s, const int32_t* n, const double* gsum,
                             const double* lse2sum, const double* hsum, float lambda, float* f,
                             float* P, float* aux, float* z, float* diag, const float* b,
                             float* b_new, float gamma, void* stream);

/*
 * moe_layer_forward -- the whole layer: route, dispatch, grouped experts, shared experts,
 * combine and statistics, enqueued on one stream with no host synchronisation.
 *   x device [T, d]; W_r device [E, d]; b device [E] fp32 or NULL
 *   W_gate, W_up device [E, M, d]; W_down device [E, d, M]
 *   Ws_gate, Ws_up device [S*M, d], Ws_down device [d, S*M]: the S shared experts stacked into one
 *   of width S*M (NULL when S == 0)
 *   y device out [T, d]
 * Optional device outputs (NULL = not returned): topk_idx [T, k] int32, topk_w [T, k] fp32,
 * counts [E] int32 (n_e), overflow [E] int32, f [E], P [E], aux [1], z [1] fp32, diag [4] fp32
 * (routing diagnostics as in moe_balance_stats), b_new [E] fp32 = the updated bias
 * (requires b; may alias b: it is written after selection), and the placement of
 * moe_dispatch ("MoE：条件计算与路由" §3): inv_perm [T, k] int32 (row of (t, j), -1 if dropped;
 * token choice only, not written under expert choice) and perm_token [moe_routed_rows(s)] int32
 * (token of each row < offsets_E; other entries unset), both 16-byte aligned.
 * Expert choice (s->routing == MOE_ROUTE_EXPERT_CHOICE; "深入理解 MoE ..." §9.2, "MoE：条件计算与
 * 路由" §路由机制的演进): expert e takes the r = min(ceil(c k T / E), T) tokens of largest logit
 * l_te (c <= 0 reads as 1; equal logits to the lower token index); token t's output sums
 * w_te E_e(x_t) over the experts that took it, in ascending e, w_te = g_te (renormalised over
 * those experts when renorm); a token no expert took gets the shared term only. b must be NULL;
 * topk_idx and topk_w are not written; counts = r, overflow = 0, f_e = n_e / (E r).
 *   saved device out of moe_saved_size(s) bytes, or NULL: the fp32 gate and up pre-activations of
 *     every kept row and of the shared experts, taken from the same accumulators as h, and the
 *     bias selected with, for a moe_layer_backward on the same inputs (training); y and every
 *     other output are the same with or without it. bf16 layers only (fp32:
 *     MOE_ERR_UNSUPPORTED); 16-byte aligned.
 *   ws device workspace of moe_workspace_size(s, MOE_CALL_LAYER) bytes
 */
moe_status moe_layer_forward(const moe_shape* s, const void* x, const void* W_r, const float* b,
                             const void* W_gate, const void* W_up, const void* W_down,
                             const void* Ws_gate, const void* Ws_up, const void* Ws_down, void* y,
                             int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* overflow,
                             float* f, float* P, float* aux, float* z, float* diag, float* b_new,
                             int32_t* inv_perm, int32_t* perm_token, float lambda, float gamma,
                             void* saved, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_layer_forward_noalloc -- moe_layer_forward for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * arguments, outputs and kernels, with the workspace taken from a static device array of
 * MOE_SCRATCH_BYTES that the library holds on each device it runs on until the process ends.
 * Nothing is allocated or freed. The array of the current device is used (the stream must belong
 * to it); its address is looked up on the first call on that device.
 * Limit: shapes with moe_workspace_size(s, MOE_CALL_LAYER) > MOE_SCRATCH_BYTES return
 * MOE_ERR_SCRATCH before anything is enqueued (e.g. the Mixtral-shaped layer, d = 4096,
 * M = 14336, E = 8, k = 2, up to about 900 tokens). No scratch contents carry over between calls
 * (every part is written before it is read). Calls on one device share its array: calls that
 * overlap in time on that device (other streams, other threads) race and must be serialised by
 * the caller. The caller still passes every input and output.
 */
#define MOE_SCRATCH_BYTES ((size_t)64 << 20)
moe_status moe_layer_forward_noalloc(const moe_shape* s, const void* x, const void* W_r,
                                     const float* b, const void* W_gate, const void* W_up,
                                     const void* W_down, const void* Ws_gate, const void* Ws_up,
                                     const void* Ws_down, void* y, int32_t* topk_idx,
                                     float* topk_w, int32_t* counts, int32_t* overflow, float* f,
                                     float* P, float* aux, float* z, float* diag, float* b_new,
                                     int32_t* inv_perm, int32_t* perm_token, float lambda,
                                     float gamma, void* saved, void* stream);

/*
 * moe_balance_loss_backward -- gradient of the layer's balance losses through the router.
 * L = aux + z_coef z, aux = lambda E sum_e f_e P_e, z = mean_t lse_t^2, as moe_balance_stats
 * computes them, with every f_e = n_e / (k T) (expert choice: n_e / (E r)) held fixed: f counts
 * discrete choices, so the gradient reaches the router through P_e and through z
 * ("MoE：条件计算与路由" §原理与演进; "MOE大模型对比篇" §2.1-§2.2). With a_e = lambda E f_e / T:
 *   softmax: dL/dl_te = g_te (a_e - sum_e' g_te' a_e') + z_coef (2/T) lse_t g_te
 *   sigmoid: dL/dl_te = s_te (1 - s_te) (a_e - sum_e' p_te' a_e') / sum_e' s_te'
 *            + z_coef (2/T) lse_t softmax(l_t)_e,   p = s / sum s
 *   dW_r = dl^T x,  dx = dl W_r.
 *   x device [T, d] (dtype); W_r device [E, d] (dtype); n device [E] int32 (the forward's loads)
 *   dlogits device out [T, E] fp32, dW_r device out [E, d] fp32, dx device out [T, d] fp32: each
 *   nullable (at least one set)
 *   ws device workspace of moe_workspace_size(s, MOE_CALL_LOSS_BACKWARD) bytes
 */
moe_status moe_balance_loss_backward(const moe_shape* s, const void* x, const void* W_r,
                                     const int32_t* n, float lambda, float z_coef,
                                     float* dlogits, float* dW_r, float* dx, void* ws,
                                     size_t ws_bytes, void* stream);

/*
 * moe_layer_backward -- gradients of <dy, y> + aux + z_coef z for the layer, with the
 * selection, the capacity cut and f held fixed (they are discrete). Recomputes the forward (the
 * same routing and placement as moe_layer_forward, the pre-activations in fp32), then:
 *   d out[row(t,j)] = w_tj dy_t, d w_tj = <dy_t, out[row(t,j)]>; gates through the
 *   renormalisation ("MoE：条件计算与路由" §7 eq. (2)) and the softmax or sigmoid to the logits,
 *   plus the balance-loss gradient of moe_balance_loss_backward; dW_r = dl^T x;
 *   per kept row (SwiGLU of "深入理解 MoE ..." §10.2): dh = d out W_down[e],
 *   dG = dh U SiLU'(G), dU = dh SiLU(G); dW_down[e] = sum d out^T h, dW_gate[e] = sum dG^T x,
 *   dW_up[e] = sum dU^T x; dx_t = (dl W_r)_t + sum_j (dG W_gate + dU W_up)_row(t,j) + shared;
 *   the shared experts take dy_t with weight 1.
 * Expert choice: the slots of token t are the experts that took it (ascending), gates
 * renormalised over them; b must be NULL (as in the forward).
 * The gradient is that of the real-valued chain (h formed in fp32 from fp32 pre-activations);
 * bf16 layers run the dx-row and weight-gradient products on bf16 MFMA with one factor of every
 * term rounded to bf16 once (dG, dU or w h); gradients are fp32.
 *   x, W_r, b, W_gate, W_up, W_down, Ws_*: as moe_layer_forward; dy device [T, d] (dtype)
 *   dx [T, d], dW_r [E, d], dW_gate, dW_up [E, M, d], dW_down [E, d, M] fp32 device out;
 *   dWs_gate, dWs_up [S*M, d], dWs_down [d, S*M] fp32 device out (required when S > 0)
 *   topk_idx device out [T, k] int32 or NULL: the token-choice selection the gradients were
 *     taken at (not written under expert choice)
 *   saved device [moe_saved_size(s) bytes] or NULL: the buffer a moe_layer_forward call on the
 *     same inputs filled; the gate/up products are then not recomputed (the routing and placement
 *     still are: they are deterministic, so the rows match). Token choice then selects with the
 *     bias kept in saved, the one the forward used, not with b: an in-place bias step between
 *     the two calls (b_new aliasing b) leaves the gradients unchanged. The gradients are
 *     bit-identical to a call without saved given the forward's bias. Read only; bf16 layers only
 *     (fp32: MOE_ERR_UNSUPPORTED); 16-byte aligned.
 *   ws device workspace of moe_workspace_size(s, MOE_CALL_LAYER_BACKWARD) bytes
 * bf16 layers read the weights in place; one expert's W_gate and W_up together (4 M d bytes), and
 * the shared experts' (4 S M d bytes), must stay under 4 GiB (MOE_ERR_UNSUPPORTED otherwise).
 */
moe_status moe_layer_backward(const moe_shape* s, const void* x, const void* W_r, const float* b,
                              const void* W_gate, const void* W_up, const void* W_down,
                              const void* Ws_gate, const void* Ws_up, const void* Ws_down,
                              const void* dy, float lambda, float z_coef, float* dx, float* dW_r,
                              float* dW_gate, float* dW_up, float* dW_down, float* dWs_gate,
                              float* dWs_up, float* dWs_down, int32_t* topk_idx,
                              const void* saved, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_set_stage_events -- profiling aid for moe_layer_forward (not a step of the method).
 * When `events` is non-NULL, later moe_layer_forward calls record events[i] (hipEvent_t handles
 * owned by the caller, count >= MOE_STAGE_COUNT) on their stream at the end of each stage:
 *   0 start, 1 route, 2 scan + placement, 3 routed gate/up GEMM (SwiGLU, rows gathered from x),
 *   4 routed down GEMM, 5 shared experts (both GEMMs), 6 combine and statistics (one launch),
 *   7 end (the interval 6..7 holds no work: the statistics are computed inside the combine launch).
 * NULL turns recording off. Process-wide setting, read and written under a lock: each forward
 * copies the handles when it starts. The caller keeps the events alive until recording is off and
 * every forward that records them has completed. A failed record makes that forward return
 * MOE_ERR_HIP (its kernels are enqueued).
 */
#define MOE_STAGE_COUNT 8
moe_status moe_set_stage_events(void* const* events, int count);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */

"""CPU oracle: the sparse MoE FFN layer forward and its balance statistics, in float64.

TEST INFRASTRUCTURE ONLY. This module is the checker, not the product: only the test suite,
the package smoke check and the benchmark's CPU-baseline leg may import or call it. It shares no
code with the HIP library (no kernels, headers, helpers or tables); both sides are fed the same
seeded inputs from the ``workloads`` module, which holds no arithmetic of the method.

It computes the plain definitions, one step per function, in the notation of the source pages:

  [ATLAS]  "MoE：条件计算与路由" (llm-knowledge-atlas.pages.dev, notes 04-04)
  [AIATTN] "深入理解 MoE (混合专家模型)：稀疏激活与高效扩展" (aiattnstudio.link)
  [CMP]    "MOE大模型对比篇" (llm.jiangnianmeng.cn)
  [CSDN]   the adg.csdn.net MoE notes page (§四 "Deepseek MoE代码")
  [T4]     "MoE" (t4mako.github.io)

The router scores the experts with a softmax over the logits (the pages' main form) or, as the
DeepSeek-V3 variant of [CSDN] §九 does, with an independent sigmoid per expert.

Readings taken where the pages are silent or disagree (each is repeated at the function that
uses it):

  * Top-k ties go to the lower expert index; slots are ordered by descending selection score.
  * The load-balancing bias b_e is added to the softmax probability g_e and used only to pick the
    experts; the gates come from the unbiased g, renormalised over the chosen set.
  * f_e = n_e / (k T), so that sum_e f_e = 1 for any k and f_e is the argmax fraction at k = 1.
  * P_e is the mean of the full (unmasked, unbiased) softmax probability.
  * Sigmoid scoring: s_te = sigmoid(l_te); the bias is added to s for selection only; the gates are
    the chosen unbiased scores renormalised over the chosen set; P_e is the mean of the scores
    normalised over all experts per token (s_te / sum_e' s_te'), which keeps sum_e P_e = 1 and
    aux = lambda under uniform routing as in the softmax case; z still uses the raw logits.
  * z = (1/T) sum_t (ln sum_e exp l_te)^2, natural log, raw logits, no coefficient.
  * Capacity C = ceil(c k T / E) evaluated in float64 as ((c * k) * T) / E; overflow is decided in
    ascending token order jointly over all k slots (first come, first kept); dropped slots add
    nothing and the surviving gates are not renormalised again.
  * Within an expert's segment, rows are in ascending token order (a stable sort by expert).
  * S shared experts take the same x as the router, are added with weight 1, and are summed.
  * Bias update: b_e <- b_e + gamma * sign(k T / E - n_e), sign(0) = 0, done in float32.
  * Expert choice: each expert takes the r tokens with the largest router logit for it (the score
    the listing ranks by), ties to the lower token index, r = C = ceil(c k T / E) (c <= 0 reads as
    c = 1), at most T; a token's gates are its scores g_te over the experts that took it,
    renormalised over that set when renorm is on; a token no expert took gets only the shared
    term. Rows of an expert are in ascending token order; loads n_e = r; the load-balancing bias
    does not apply (a per-expert shift leaves every expert's ranking of tokens unchanged).
  * Loss backward: the gradient of L = aux + z_coef * z with respect to the logits, W_r and x,
    with every f_e held fixed (it counts discrete selections, so no gradient flows through it;
    the gradient reaches the router through P_e and the z-loss).
  * Diagnostics: routing entropy is the token mean of H(p_t) = -sum_e p_te ln p_te (natural log,
    0 ln 0 = 0) of the same per-token distribution P_e averages; the load Gini coefficient is
    sum_ij |n_i - n_j| / (2 E sum_e n_e); max/mean load is max_e n_e / (sum_e n_e / E); the
    importance CV^2 uses the population variance of Importance_e = sum_t p_te.

Every function here is pinned by the CPU tests against closed forms, invariants, brute force or an
independent formula from the pages.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np


def _f64(a) -> np.ndarray:
    """Host float64 copy of an array or torch tensor (bf16 inputs are upcast exactly)."""
    if hasattr(a, "detach"):
        a = a.detach().to("cpu")
        if str(a.dtype) == "torch.bfloat16":
            a = a.float()
        a = a.numpy()
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------------------------
# Router: [ATLAS] §原理与演进 "Router 如何让参数多、每 token 计算少": g(x) = softmax(W_r x)
# ---------------------------------------------------------------------------------------------

def router_logits(x: np.ndarray, W_r: np.ndarray) -> np.ndarray:
    """l[t, e] = sum_i x[t, i] * W_r[e, i]  (the router projection W_r x, no bias term). [T, E]"""
    return _f64(x) @ _f64(W_r).T


def softmax_lse(l: np.ndarray):
    """Max-subtracted softmax over experts and its log-sum-exp.

    m_t = max_e l_te;  lse_t = m_t + ln sum_e exp(l_te - m_t);  g_te = exp(l_te - lse_t).
    The max subtraction is the stability device of [T4] §训练不稳定 (2. 舍入误差); lse_t is the
    inner term of the router z-loss of [CMP] §2.2.
    Returns (g [T, E], lse [T]).
    """
    l = _f64(l)
    m = l.max(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(l - m).sum(axis=1))
    g = np.exp(l - lse[:, None])
    return g, lse


def sigmoid_scores(l: np.ndarray) -> np.ndarray:
    """s_te = 1 / (1 + exp(-l_te)): every expert scored on its own, with no sum over experts
    ([CSDN] §九, why DeepSeek-V3 moved its gate from softmax to sigmoid). [T, E]"""
    l = _f64(l)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-l))


def score_distribution(g: np.ndarray, scoring: str = "softmax") -> np.ndarray:
    """Per-token distribution over experts whose mean is P_e: the softmax probabilities
    themselves, or the sigmoid scores divided by their sum over all experts. [T, E]"""
    g = _f64(g)
    if scoring == "softmax":
        return g
    if scoring == "sigmoid":
        return g / g.sum(axis=1, keepdims=True)
    raise ValueError(f"unknown scoring {scoring!r}")


def selection_scores(g: np.ndarray, b: Optional[np.ndarray]) -> np.ndarray:
    """s_te = g_te + b_e ([ATLAS] §无辅助损失负载均衡（ALF-LB）: the per-expert bias is applied to
    the routing score before Top-K); s = g when there is no bias."""
    g = _f64(g)
    if b is None:
        return g.copy()
    return g + _f64(b)[None, :]


def top_k(s: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest s_te per token, ordered by descending score, ties to the lower
    expert index ([ATLAS] §7 eq. (1) S = TopK(g(x))). A stable sort of -s along experts keeps
    equal scores in ascending index order. [T, k] int64."""
    s = _f64(s)
    order = np.argsort(-s, axis=1, kind="stable")
    return order[:, :k].astype(np.int64)


def topk_margin(s: np.ndarray, k: int) -> np.ndarray:
    """Gap between the k-th and (k+1)-th largest selection score per token (inf when k == E)."""
    s = _f64(s)
    if k >= s.shape[1]:
        return np.full(s.shape[0], np.inf)
    srt = -np.sort(-s, axis=1)
    return srt[:, k - 1] - srt[:, k]


def gate_weights(g: np.ndarray, S: np.ndarray, renorm: bool = True) -> np.ndarray:
    """Gates of the chosen experts from the UNBIASED g: w_tj = g[t, S_tj], divided by
    sum_j' g[t, S_tj'] when renormalising ([ATLAS] §7 eq. (2) g~_e = g_e / sum_{j in S} g_j).
    [T, k]"""
    g = _f64(g)
    w = np.take_along_axis(g, S, axis=1)
    if renorm:
        w = w / w.sum(axis=1, keepdims=True)
    return w


# ---------------------------------------------------------------------------------------------
# Loads and capacity: [ATLAS] §1 (n_e) and §3 (C = ceil(c B k / E))
# ---------------------------------------------------------------------------------------------

def expert_loads(S: np.ndarray, E: int) -> np.ndarray:
    """n_e = sum_t 1[e in S_t] ([ATLAS] §1 "容量与激活计算为什么能分离"), before capacity. [E] int64"""
    n = np.zeros(E, dtype=np.int64)
    for e in S.reshape(-1):
        n[int(e)] += 1
    return n


def capacity(c: Optional[float], k: int, T: int, E: int) -> Optional[int]:
    """C = ceil(c B k / E) of [ATLAS] §3 (B = T tokens), in float64 as ((c*k)*T)/E with c taken as
    the float32 value the caller passes. None (no limit) when c is None or c <= 0."""
    if c is None:
        return None
    c32 = float(np.float32(c))
    if c32 <= 0.0:
        return None
    return int(math.ceil(((c32 * k) * T) / E))


def expert_choice(l: np.ndarray, r: int) -> np.ndarray:
    """Expert-choice selection ([AIATTN] §9.2 Expert Choice MoE: every expert picks the top tokens
    by its score column; [ATLAS] §路由机制的演进, experts choose top-r_e tokens): for each expert, the
    r tokens of largest l[t, e] (a stable sort of -l down the column keeps equal scores in
    ascending token order), returned in ascending token order. [E, r] int64"""
    l = _f64(l)
    order = np.argsort(-l, axis=0, kind="stable")
    return np.sort(order[:r, :].T, axis=1).astype(np.int64)


def expert_choice_capacity(c: Optional[float], k: int, T: int, E: int) -> int:
    """r = ceil(c k T / E) as for token choice, with c <= 0 (or None) read as 1, at most T."""
    C = capacity(c, k, T, E)
    if C is None:
        C = capacity(1.0, k, T, E)
    return min(C, T)


def dispatch(S: np.ndarray, E: int, C: Optional[int]):
    """Expert-contiguous placement of the (token, slot) assignments with capacity dropping.

    For expert e, the tokens that chose it are listed in ascending token order; the assignment's
    position p(t, e) is its index in that list and it is kept iff p < C. Kept assignments of e fill
    rows off_e .. off_e + kept_e - 1 in that order, off_e = sum_{e' < e} kept_e'. This follows the
    token-major flattening and per-expert truncation of [CSDN] §四 (the demo MoE's expert loop
    with its capacity check) and the histogram-then-sort placement of its DeepseekV3MoE.moe_infer.

    Returns dict with pos [T,k], row [T,k] (-1 = dropped), kept [E], overflow [E], offsets [E+1],
    perm_token [P_kept].
    """
    T, k = S.shape
    lists = [[] for _ in range(E)]          # (t, j) in ascending t for each expert
    for t in range(T):
        for j in range(k):
            lists[int(S[t, j])].append((t, j))
    pos = np.full((T, k), -1, dtype=np.int64)
    kept = np.zeros(E, dtype=np.int64)
    for e in range(E):
        for p, (t, j) in enumerate(lists[e]):
            pos[t, j] = p
        kept[e] = len(lists[e]) if C is None else min(len(lists[e]), C)
    n = np.array([len(l) for l in lists], dtype=np.int64)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(kept)
    row = np.full((T, k), -1, dtype=np.int64)
    perm_token = np.full(int(offsets[-1]), -1, dtype=np.int64)
    for e in range(E):
        for p, (t, j) in enumerate(lists[e]):
            if p < kept[e]:
                r = offsets[e] + p
                row[t, j] = r
                perm_token[r] = t
    return {"pos": pos, "row": row, "kept": kept, "overflow": n - kept,
            "offsets": offsets, "perm_token": perm_token}


# ---------------------------------------------------------------------------------------------
# Experts: [AIATTN] §10.2 与 SwiGLU 的结合 / §11: SwiGLU(x) = SiLU(W_1 x) ⊙ (W_3 x), then W_2
# ---------------------------------------------------------------------------------------------

def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z / (1 + exp(-z))."""
    z = _f64(z)
    return z / (1.0 + np.exp(-z))


def swiglu_expert(X: np.ndarray, W_gate: np.ndarray, W_up: np.ndarray, W_down: np.ndarray) -> np.ndarray:
    """E_e(X) = W_down (SiLU(W_gate X) ⊙ (W_up X)) for rows X [n, d]; W_gate, W_up [M, d]
    (W_1 and W_3 of the page), W_down [d, M] (W_2); no biases. Returns [n, d]."""
    X = _f64(X)
    G = X @ _f64(W_gate).T
    U = X @ _f64(W_up).T
    h = silu(G) * U
    return h @ _f64(W_down).T


def shared_experts(x: np.ndarray, shared: Sequence) -> np.ndarray:
    """sum_s E^s(x) over the S shared experts, each applied to every token with weight 1
    ([CMP] §3.3 shared-expert isolation; [CSDN] §四 DeepseekV3MoE adds shared_experts(identity)
    to the routed output)."""
    x = _f64(x)
    out = np.zeros_like(x)
    for Wg, Wu, Wd in shared:
        out += swiglu_expert(x, Wg, Wu, Wd)
    return out


def combine(T: int, d: int, row: np.ndarray, w: np.ndarray, out_perm: np.ndarray,
            shared_out: Optional[np.ndarray] = None) -> np.ndarray:
    """y_t = sum_{j : row_tj >= 0} w_tj * out_perm[row_tj] (+ shared_t)  ([ATLAS] §7 eq. (3))."""
    y = np.zeros((T, d)) if shared_out is None else _f64(shared_out).copy()
    for t in range(T):
        for j in range(row.shape[1]):
            r = int(row[t, j])
            if r >= 0:
                y[t] += w[t, j] * out_perm[r]
    return y


# ---------------------------------------------------------------------------------------------
# Balance statistics and the loss-free-balancing bias update
# ---------------------------------------------------------------------------------------------

def balance_stats(n: np.ndarray, g: np.ndarray, lse: np.ndarray, k: int, lam: float):
    """f_e = n_e / (k T);  P_e = (1/T) sum_t g_te;  aux = lambda * E * sum_e f_e P_e
    ([ATLAS] §原理与演进, L_balance = lambda E sum_e f_e P_e; [AIATTN] §4.2.1; [CMP] §2.1);
    z = (1/T) sum_t lse_t^2 ([CMP] §2.2 z-loss L_z). g is the per-token distribution of
    score_distribution. Returns dict of float64 values."""
    g = _f64(g)
    T, E = g.shape
    f = _f64(n) / float(k * T)
    P = g.sum(axis=0) / float(T)
    aux = float(lam) * E * float((f * P).sum())
    z = float((_f64(lse) ** 2).sum() / float(T))
    return {"f": f, "P": P, "aux": aux, "z": z}


def balance_loss_grad_logits(l: np.ndarray, f: np.ndarray, lam: float, z_coef: float,
                             scoring: str = "softmax") -> np.ndarray:
    """dL/dl for L = aux + z_coef z, aux = lambda E sum_e f_e P_e, P_e = (1/T) sum_t p_te,
    z = (1/T) sum_t lse_t^2, with f held fixed ([ATLAS] §原理与演进: f_e is a count and the
    gradient flows through P_e; [CMP] §2.2 z-loss). With a_e = lambda E f_e / T:
      softmax p = g:          dL/dl_te = g_te (a_e - sum_e' g_te' a_e') + z_coef (2/T) lse_t g_te
      sigmoid p = s / sum s:  dL/dl_te = s_te (1 - s_te) (a_e - sum_e' p_te' a_e') / sum_e' s_te'
                              + z_coef (2/T) lse_t softmax(l_t)_e   [T, E]"""
    l = _f64(l)
    T, E = l.shape
    a = float(lam) * E * _f64(f) / T
    g, lse = softmax_lse(l)
    dz = float(z_coef) * (2.0 / T) * lse[:, None] * g
    if scoring == "softmax":
        return g * (a[None, :] - (g * a[None, :]).sum(axis=1, keepdims=True)) + dz
    if scoring == "sigmoid":
        s = sigmoid_scores(l)
        S = s.sum(axis=1, keepdims=True)
        p = s / S
        return s * (1.0 - s) * (a[None, :] - (p * a[None, :]).sum(axis=1, keepdims=True)) / S + dz
    raise ValueError(f"unknown scoring {scoring!r}")


def balance_loss_backward(x, W_r, f, lam: float, z_coef: float, scoring: str = "softmax"):
    """Router gradients of L: dl (as above), dW_r = dl^T x [E, d], dx = dl W_r [T, d]."""
    x64 = _f64(x)
    W64 = _f64(W_r)
    dl = balance_loss_grad_logits(router_logits(x64, W64), f, lam, z_coef, scoring)
    return {"dlogits": dl, "dW_r": dl.T @ x64, "dx": dl @ W64}


def silu_grad(z: np.ndarray) -> np.ndarray:
    """d SiLU / dz = sigma(z) (1 + z (1 - sigma(z)))."""
    z = _f64(z)
    sg = 1.0 / (1.0 + np.exp(-z))
    return sg * (1.0 + z * (1.0 - sg))


def layer_backward(x, W_r, W_gate, W_up, W_down, dy, k: int, b=None, shared=(), c=None,
                   renorm: bool = True, lam: float = 0.01, z_coef: float = 0.0,
                   scoring: str = "softmax", topk_idx=None, magnitudes: bool = False):
    """Gradients of <dy, y> + aux + z_coef z with respect to x, W_r and every expert weight, for
    the token-choice layer of layer_forward (selection, capacity and f held fixed: they are
    discrete). The chain, step by step:
      d out[row(t,j)] = w_tj dy_t;   d w_tj = <dy_t, out[row(t,j)]>   (kept slots; dropped add 0)
      gates: w_j = g_j / sum_S g (renorm) -> dg_e = (dw_e - sum_j w_j dw_j) / sum_S g, else dg = dw
      scores: softmax dl = g (dg - sum_e g dg); sigmoid dl = s (1 - s) dg; plus the balance-loss
      gradient (balance_loss_grad_logits); dW_r = dl^T x, dx += dl W_r
      per kept row: dh = d out W_down; dW_down += d out^T h; dG = dh U SiLU'(G), dU = dh SiLU(G);
      dx_t += dG W_gate + dU W_up; dW_gate += dG^T x_t, dW_up += dU^T x_t
      shared experts: the same with d out = dy_t and weight 1.
    Returns dict of float64 arrays. With magnitudes=True, out["magnitude"] holds, for dx, dW_r and
    every weight gradient, the sum of the absolute values of the terms the gradient is a sum of
    (the same products taken over |.|): the scale of the rounding bound of any evaluation that
    rounds one factor of each term."""
    x64 = _f64(x)
    T, d = x64.shape
    r = route(x64, W_r, k, b, renorm, scoring)
    l, g = r["logits"], r["g"]
    E = g.shape[1]
    S = r["topk_idx"] if topk_idx is None else np.asarray(topk_idx, dtype=np.int64)
    w = gate_weights(g, S, renorm)
    n = expert_loads(S, E)
    dsp = dispatch(S, E, capacity(c, k, T, E))
    dy64 = _f64(dy)
    out = {"dx": np.zeros((T, d)), "dW_gate": np.zeros_like(_f64(W_gate)),
           "dW_up": np.zeros_like(_f64(W_up)), "dW_down": np.zeros_like(_f64(W_down))}
    dw = np.zeros((T, k))
    mag = {key: np.zeros_like(val) for key, val in out.items()}
    for e in range(E):
        rows = [(int(dsp["offsets"][e]) + p, int(dsp["perm_token"][dsp["offsets"][e] + p]))
                for p in range(int(dsp["kept"][e]))]
        if not rows:
            continue
        Wg, Wu, Wd = _f64(W_gate[e]), _f64(W_up[e]), _f64(W_down[e])
        toks = [t for _, t in rows]
        X = x64[toks]
        G = X @ Wg.T
        U = X @ Wu.T
        h = silu(G) * U
        O = h @ Wd.T
        # the slot of each row, for its gate
        slot = np.array([int(np.nonzero(dsp["row"][t] == rr)[0][0]) for rr, t in rows])
        wt = w[toks, slot]
        dO = wt[:, None] * dy64[toks]
        dw[toks, slot] = (dy64[toks] * O).sum(axis=1)
        dh = dO @ Wd
        out["dW_down"][e] = dO.T @ h
        dG = dh * U * silu_grad(G)
        dU = dh * silu(G)
        out["dW_gate"][e] = dG.T @ X
        out["dW_up"][e] = dU.T @ X
        np.add.at(out["dx"], toks, dG @ Wg + dU @ Wu)
        if magnitudes:
            mag["dW_down"][e] = np.abs(dO).T @ np.abs(h)
            mag["dW_gate"][e] = np.abs(dG).T @ np.abs(X)
            mag["dW_up"][e] = np.abs(dU).T @ np.abs(X)
            np.add.at(mag["dx"], toks, np.abs(dG) @ np.abs(Wg) + np.abs(dU) @ np.abs(Wu))
    # router: gates -> scores -> logits
    dg = np.zeros((T, E))
    gS = np.take_along_axis(g, S, axis=1)
    if renorm:
        den = gS.sum(axis=1, keepdims=True)
        dgS = (dw - (w * dw).sum(axis=1, keepdims=True)) / den
    else:
        dgS = dw
    np.put_along_axis(dg, S, dgS, axis=1)
    if scoring == "softmax":
        dl = g * (dg - (g * dg).sum(axis=1, keepdims=True))
    else:
        dl = g * (1.0 - g) * dg
    f = n / float(k * T)
    dl = dl + balance_loss_grad_logits(l, f, lam, z_coef, scoring)
    W64 = _f64(W_r)
    out["dW_r"] = dl.T @ x64
    out["dx"] += dl @ W64
    out["dlogits"] = dl
    if magnitudes:
        mag["dW_r"] = np.abs(dl).T @ np.abs(x64)
        mag["dx"] += np.abs(dl) @ np.abs(W64)
    sh_grads, sh_mag = [], []
    for Wg, Wu, Wd in shared:
        Wg, Wu, Wd = _f64(Wg), _f64(Wu), _f64(Wd)
        G = x64 @ Wg.T
        U = x64 @ Wu.T
        h = silu(G) * U
        dh = dy64 @ Wd
        dG = dh * U * silu_grad(G)
        dU = dh * silu(G)
        out["dx"] += dG @ Wg + dU @ Wu
        sh_grads.append((dG.T @ x64, dU.T @ x64, dy64.T @ h))
        if magnitudes:
            mag["dx"] += np.abs(dG) @ np.abs(Wg) + np.abs(dU) @ np.abs(Wu)
            ax = np.abs(x64)
            sh_mag.append((np.abs(dG).T @ ax, np.abs(dU).T @ ax, np.abs(dy64).T @ np.abs(h)))
    out["shared"] = sh_grads
    if magnitudes:
        mag["shared"] = sh_mag
        out["magnitude"] = mag
    out["topk_idx"] = S
    return out


def layer_backward_expert_choice(x, W_r, W_gate, W_up, W_down, dy, k: int, shared=(), c=None,
                                 renorm: bool = True, lam: float = 0.01, z_coef: float = 0.0,
                                 scoring: str = "softmax", chosen=None, magnitudes: bool = False):
    """Gradients of <dy, y> + aux + z_coef z for the expert-choice layer of
    layer_forward_expert_choice, with the selection (each expert's r tokens) held fixed. The chain
    is that of layer_backward with the set of experts that took token t, E_t, in place of the top-k
    slots:
      d w_te = <dy_t, E_e(x_t)> for e in E_t;  renorm: dg_te = (d w_te - sum_{E_t} w dw) / sum_{E_t} g,
      else dg_te = d w_te;  then the softmax / sigmoid chain to the logits, plus the balance-loss
      gradient with f_e = n_e / sum n = 1/E held fixed; per expert row: d out = w_te dy_t, etc.
    ``chosen`` (optional, [E, r]) replaces the oracle's own selection. Returns float64 arrays (and
    "magnitude" as in layer_backward)."""
    x64 = _f64(x)
    dy64 = _f64(dy)
    T, d = x64.shape
    r_ = route(x64, W_r, 1, None, renorm, scoring)
    l, g = r_["logits"], r_["g"]
    E = g.shape[1]
    r = expert_choice_capacity(c, k, T, E)
    chosen = expert_choice(l, r) if chosen is None else np.asarray(chosen, dtype=np.int64)
    member = np.zeros((T, E), dtype=bool)
    for e in range(E):
        member[chosen[e], e] = True
    gm = np.where(member, g, 0.0)
    den = gm.sum(axis=1)
    if renorm:
        w = np.divide(gm, den[:, None], out=np.zeros_like(gm), where=den[:, None] > 0)
    else:
        w = gm
    out = {"dx": np.zeros((T, d)), "dW_gate": np.zeros_like(_f64(W_gate)),
           "dW_up": np.zeros_like(_f64(W_up)), "dW_down": np.zeros_like(_f64(W_down))}
    mag = {key: np.zeros_like(val) for key, val in out.items()}
    dw = np.zeros((T, E))
    for e in range(E):
        toks = chosen[e]
        if len(toks) == 0:
            continue
        Wg, Wu, Wd = _f64(W_gate[e]), _f64(W_up[e]), _f64(W_down[e])
        X = x64[toks]
        G, U = X @ Wg.T, X @ Wu.T
        h = silu(G) * U
        O = h @ Wd.T
        wt = w[toks, e]
        dO = wt[:, None] * dy64[toks]
        dw[toks, e] = (dy64[toks] * O).sum(axis=1)
        dh = dO @ Wd
        dG, dU = dh * U * silu_grad(G), dh * silu(G)
        out["dW_down"][e] = dO.T @ h
        out["dW_gate"][e] = dG.T @ X
        out["dW_up"][e] = dU.T @ X
        out["dx"][toks] += dG @ Wg + dU @ Wu
        if magnitudes:
            mag["dW_down"][e] = np.abs(dO).T @ np.abs(h)
            mag["dW_gate"][e] = np.abs(dG).T @ np.abs(X)
            mag["dW_up"][e] = np.abs(dU).T @ np.abs(X)
            mag["dx"][toks] += np.abs(dG) @ np.abs(Wg) + np.abs(dU) @ np.abs(Wu)
    # router: gates over E_t -> scores -> logits
    if renorm:
        dg = np.where(member, (dw - (w * dw).sum(axis=1, keepdims=True)), 0.0)
        dg = np.divide(dg, den[:, None], out=np.zeros_like(dg), where=den[:, None] > 0)
    else:
        dg = np.where(member, dw, 0.0)
    if scoring == "softmax":
        dl = g * (dg - (g * dg).sum(axis=1, keepdims=True))
    else:
        dl = g * (1.0 - g) * dg
    n = np.full(E, r, dtype=np.int64)
    dl = dl + balance_loss_grad_logits(l, n / float(n.sum()), lam, z_coef, scoring)
    W64 = _f64(W_r)
    out["dW_r"] = dl.T @ x64
    out["dx"] += dl @ W64
    out["dlogits"] = dl
    if magnitudes:
        mag["dW_r"] = np.abs(dl).T @ np.abs(x64)
        mag["dx"] += np.abs(dl) @ np.abs(W64)
    sh_grads, sh_mag = [], []
    for Wg, Wu, Wd in shared:
        Wg, Wu, Wd = _f64(Wg), _f64(Wu), _f64(Wd)
        G, U = x64 @ Wg.T, x64 @ Wu.T
        h = silu(G) * U
        dh = dy64 @ Wd
        dG, dU = dh * U * silu_grad(G), dh * silu(G)
        out["dx"] += dG @ Wg + dU @ Wu
        sh_grads.append((dG.T @ x64, dU.T @ x64, dy64.T @ h))
        if magnitudes:
            mag["dx"] += np.abs(dG) @ np.abs(Wg) + np.abs(dU) @ np.abs(Wu)
            ax = np.abs(x64)
            sh_mag.append((np.abs(dG).T @ ax, np.abs(dU).T @ ax, np.abs(dy64).T @ np.abs(h)))
    out["shared"] = sh_grads
    out["chosen"] = chosen
    if magnitudes:
        mag["shared"] = sh_mag
        out["magnitude"] = mag
    return out


def layer_backward_sampled(x, W_r, W_gate, W_up, W_down, dy, k: int, b=None, shared=(), c=None,
                           renorm: bool = True, lam: float = 0.01, z_coef: float = 0.0,
                           scoring: str = "softmax", topk_idx=None, tokens=(), expert_cols=(),
                           shared_cols=(), expert_weights=None):
    """Selected entries of layer_backward, each evaluated on its own from the same chain, for
    layers too large for the whole backward on the host:
      dx[t] for t in tokens (its kept slots' experts, its router row and the shared experts);
      for (e, m) in expert_cols: row m of dW_gate[e] and of dW_up[e] (sums over e's kept rows r of
        dG[r, m] x_t(r), dU[r, m] x_t(r)) and column m of dW_down[e] (sum over r of
        w_r dy_t(r) h[r, m]) -- G[r, m], U[r, m] and P[r, m] = dy_t(r) W_down[e][:, m] are single
        dot products, so a column costs O(rows d);
      for m in shared_cols: row m of the stacked shared gate/up gradients and column m of the
        stacked down gradient (the S experts of width M side by side).
    Routing, loads and the balance-loss gradient are computed for all tokens. ``expert_weights``
    (optional) is a callable e -> (W_gate_e, W_up_e, W_down_e). Returns float64 arrays with the
    magnitudes (sums of |terms|) of every entry under "magnitude"."""
    x64 = _f64(x)
    dy64 = _f64(dy)
    T, d = x64.shape
    r = route(x64, W_r, k, b, renorm, scoring)
    l, g = r["logits"], r["g"]
    E = g.shape[1]
    S = r["topk_idx"] if topk_idx is None else np.asarray(topk_idx, dtype=np.int64)
    w = gate_weights(g, S, renorm)
    n = expert_loads(S, E)
    dsp = dispatch(S, E, capacity(c, k, T, E))
    bl = balance_loss_grad_logits(l, n / float(k * T), lam, z_coef, scoring)
    W64 = _f64(W_r)
    weights = expert_weights if expert_weights is not None else (
        lambda e: (W_gate[e], W_up[e], W_down[e]))
    tokens = [int(t) for t in tokens]
    out = {"dx": np.zeros((len(tokens), d)), "magnitude": {"dx": np.zeros((len(tokens), d))}}
    # ---- dx of the sampled tokens: expert part per kept slot, grouped by expert
    slots = {}
    for i, t in enumerate(tokens):
        for j in range(k):
            if dsp["row"][t, j] >= 0:
                slots.setdefault(int(S[t, j]), []).append((i, t, j))
    dw = np.zeros((len(tokens), k))
    for e, lst in sorted(slots.items()):
        Wg, Wu, Wd = (_f64(a) for a in weights(e))
        for i, t, j in lst:
            G, U = Wg @ x64[t], Wu @ x64[t]
            P = dy64[t] @ Wd
            dw[i, j] = P @ (silu(G) * U)
            dh = w[t, j] * P
            dG, dU = dh * U * silu_grad(G), dh * silu(G)
            out["dx"][i] += dG @ Wg + dU @ Wu
            out["magnitude"]["dx"][i] += np.abs(dG) @ np.abs(Wg) + np.abs(dU) @ np.abs(Wu)
    # router part: gates -> scores -> logits, plus the balance-loss gradient
    for i, t in enumerate(tokens):
        gt = g[t]
        dg = np.zeros(E)
        if renorm:
            dg[S[t]] = (dw[i] - (w[t] * dw[i]).sum()) / gt[S[t]].sum()
        else:
            dg[S[t]] = dw[i]
        dl = gt * (dg - (gt * dg).sum()) if scoring == "softmax" else gt * (1.0 - gt) * dg
        dl = dl + bl[t]
        out["dx"][i] += dl @ W64
        out["magnitude"]["dx"][i] += np.abs(dl) @ np.abs(W64)
    for Wg, Wu, Wd in shared:
        Wg, Wu, Wd = _f64(Wg), _f64(Wu), _f64(Wd)
        for i, t in enumerate(tokens):
            G, U = Wg @ x64[t], Wu @ x64[t]
            dh = dy64[t] @ Wd
            dG, dU = dh * U * silu_grad(G), dh * silu(G)
            out["dx"][i] += dG @ Wg + dU @ Wu
            out["magnitude"]["dx"][i] += np.abs(dG) @ np.abs(Wg) + np.abs(dU) @ np.abs(Wu)
    # ---- weight-gradient entries of the routed experts
    for key in ("dW_gate", "dW_up", "dW_down"):
        out[key], out["magnitude"][key] = [], []
    for e, m in expert_cols:
        e, m = int(e), int(m)
        rows = range(int(dsp["offsets"][e]), int(dsp["offsets"][e + 1]))
        toks = np.array([int(dsp["perm_token"][rr]) for rr in rows], dtype=np.int64)
        slot = np.array([int(np.nonzero(dsp["row"][t] == rr)[0][0]) for rr, t in zip(rows, toks)],
                        dtype=np.int64)
        Wg, Wu, Wd = weights(e)
        X, Y = x64[toks], dy64[toks]
        G, U = X @ _f64(Wg[m]), X @ _f64(Wu[m])
        wt = w[toks, slot] if len(toks) else np.zeros(0)
        dh = wt * (Y @ _f64(Wd[:, m]))
        dG, dU, h = dh * U * silu_grad(G), dh * silu(G), silu(G) * U
        dO = wt[:, None] * Y
        for key, val, mag in (("dW_gate", dG @ X, np.abs(dG) @ np.abs(X)),
                              ("dW_up", dU @ X, np.abs(dU) @ np.abs(X)),
                              ("dW_down", dO.T @ h, np.abs(dO).T @ np.abs(h))):
            out[key].append(val)
            out["magnitude"][key].append(mag)
    # ---- shared experts: column m of the stacked width S M
    for key in ("dWs_gate", "dWs_up", "dWs_down"):
        out[key], out["magnitude"][key] = [], []
    for m in shared_cols:
        m = int(m)
        Wg, Wu, Wd = shared[m // shared[0][0].shape[0]]
        mm = m % shared[0][0].shape[0]
        G, U = x64 @ _f64(Wg[mm]), x64 @ _f64(Wu[mm])
        dh = dy64 @ _f64(Wd[:, mm])
        dG, dU, h = dh * U * silu_grad(G), dh * silu(G), silu(G) * U
        for key, val, mag in (("dWs_gate", dG @ x64, np.abs(dG) @ np.abs(x64)),
                              ("dWs_up", dU @ x64, np.abs(dU) @ np.abs(x64)),
                              ("dWs_down", dy64.T @ h, np.abs(dy64).T @ np.abs(h))):
            out[key].append(val)
            out["magnitude"][key].append(mag)
    out["topk_idx"] = S
    out["tokens"] = np.array(tokens, dtype=np.int64)
    return out


def routing_entropy(probs: np.ndarray) -> float:
    """Mean over tokens of H(g(x)) = -sum_e g_e ln g_e ([ATLAS] §9 专业化是否真的发生: the routing
    entropy describes how concentrated the choice is), with 0 ln 0 = 0."""
    p = _f64(probs)
    with np.errstate(divide="ignore", invalid="ignore"):
        terms = np.where(p > 0.0, p * np.log(p), 0.0)
    return float(-terms.sum(axis=1).mean())


def load_gini(n: np.ndarray) -> float:
    """Gini coefficient of the expert loads ([ATLAS] §10 MoE 评估的标准化: the load distribution
    by its Gini coefficient or the max/mean ratio): sum_i sum_j |n_i - n_j| / (2 E sum_e n_e)."""
    x = _f64(n)
    E = x.shape[0]
    tot = x.sum()
    if tot == 0.0:
        return 0.0
    return float(np.abs(x[:, None] - x[None, :]).sum() / (2.0 * E * tot))


def load_max_over_mean(n: np.ndarray) -> float:
    """max_e n_e / mean_e n_e ([ATLAS] §10; the critical path waits for the busiest expert, §8)."""
    x = _f64(n)
    mean = x.sum() / x.shape[0]
    return float(x.max() / mean) if mean > 0.0 else 0.0


def importance_cv2(importance: np.ndarray) -> float:
    """CV(Importance)^2 = Var / Mean^2 of Importance_e = sum_t G_e(x_t) ([CSDN] 平衡专家利用率:
    the importance loss is w_importance times this square), population variance."""
    x = _f64(importance)
    mean = x.mean()
    return float(((x - mean) ** 2).mean() / (mean * mean)) if mean != 0.0 else 0.0


def diagnostics(n: np.ndarray, probs: np.ndarray) -> dict:
    """Routing entropy, load Gini, max/mean load and importance CV^2 of one batch."""
    p = _f64(probs)
    return {"entropy": routing_entropy(p), "gini": load_gini(n),
            "max_over_mean": load_max_over_mean(n), "importance_cv2": importance_cv2(p.sum(axis=0))}


def bias_update(b: np.ndarray, n: np.ndarray, k: int, T: int, gamma: float) -> np.ndarray:
    """b_e <- b_e + gamma * sign(k T / E - n_e) in float32: an overloaded expert's bias goes down,
    an underloaded one's goes up ([ATLAS] §无辅助损失负载均衡（ALF-LB）), sign(0) = 0."""
    b32 = np.asarray(b, dtype=np.float32)
    E = b32.shape[0]
    mean_load = (k * T) / E
    sgn = np.sign(mean_load - _f64(n)).astype(np.float32)
    return (b32 + np.float32(gamma) * sgn).astype(np.float32)


# ---------------------------------------------------------------------------------------------
# The whole layer
# ---------------------------------------------------------------------------------------------

def route(x, W_r, k: int, b=None, renorm: bool = True, scoring: str = "softmax"):
    """Router stage for all tokens: logits, scores (softmax or per-expert sigmoid), selection,
    gates and margins. lse always comes from the raw logits (z-loss)."""
    l = router_logits(x, W_r)
    g, lse = softmax_lse(l)
    if scoring == "sigmoid":
        g = sigmoid_scores(l)
    elif scoring != "softmax":
        raise ValueError(f"unknown scoring {scoring!r}")
    s = selection_scores(g, b)
    S = top_k(s, k)
    w = gate_weights(g, S, renorm)
    return {"logits": l, "g": g, "lse": lse, "s": s, "topk_idx": S, "topk_w": w,
            "margin": topk_margin(s, k), "probs": score_distribution(g, scoring)}


def layer_forward_expert_choice(x, W_r, W_gate, W_up, W_down, k: int, shared=(), c=None,
                                renorm: bool = True, lam: float = 0.01, tokens=None,
                                expert_weights=None, scoring: str = "softmax",
                                magnitudes: bool = False):
    """Expert-choice layer: expert e applies E_e to the r tokens it chose; y_t sums w_te E_e(x_t)
    over the experts that chose t, in ascending expert order, plus the shared experts.
    ``magnitudes``: res["magnitude"] as in layer_forward (sums of |terms| per element of y)."""
    x64 = _f64(x)
    T, d = x64.shape
    r_ = route(x64, W_r, 1, None, renorm, scoring)
    l, g = r_["logits"], r_["g"]
    E = g.shape[1]
    r = expert_choice_capacity(c, k, T, E)
    chosen = expert_choice(l, r)
    member = np.zeros((T, E), dtype=bool)
    for e in range(E):
        member[chosen[e], e] = True
    w = np.where(member, g, 0.0)
    if renorm:
        den = w.sum(axis=1, keepdims=True)
        w = np.divide(w, den, out=np.zeros_like(w), where=den > 0)
    n = np.full(E, r, dtype=np.int64)
    want = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    y = np.zeros((len(want), d))
    xs = x64[want]
    if shared:
        y += shared_experts(xs, shared)
    mag = np.zeros((len(want), d)) if magnitudes else None
    if magnitudes:
        for Ws in shared:
            mag += np.abs(swiglu_expert(xs, *Ws))
    pos = {int(t): i for i, t in enumerate(want)}
    for e in range(E):
        rows = [int(t) for t in chosen[e] if int(t) in pos]
        if not rows:
            continue
        We = expert_weights(e) if expert_weights is not None else (W_gate[e], W_up[e], W_down[e])
        O = swiglu_expert(x64[rows], *We)
        for i, t in enumerate(rows):
            y[pos[t]] += w[t, e] * O[i]
            if magnitudes:
                mag[pos[t]] += np.abs(w[t, e] * O[i])
    # f_e = n_e / sum_e n_e (equal loads: 1 / E), P_e from the same distribution as token choice
    f = n / float(n.sum())
    P = r_["probs"].sum(axis=0) / float(T)
    aux = float(lam) * E * float((f * P).sum())
    z = float((r_["lse"] ** 2).sum() / float(T))
    return {"y": y, "magnitude": mag, "tokens": want, "chosen": chosen, "r": r, "w": w, "n": n,
            "f": f, "P": P,
            "aux": aux, "z": z, "lse": r_["lse"], "g": g, "logits": l,
            "diag": diagnostics(n, r_["probs"]),
            "uncovered": int((~member.any(axis=1)).sum())}


def layer_forward(x, W_r, W_gate, W_up, W_down, k: int, b=None, shared=(), c=None,
                  renorm: bool = True, lam: float = 0.01, gamma: float = 1e-3,
                  topk_idx=None, tokens=None, expert_weights=None, scoring: str = "softmax",
                  magnitudes: bool = False):
    """y = sum_{e in S_t} w_te E_e(x_t) + sum_s E^s(x_t), plus loads, drops and statistics.

    ``topk_idx`` (optional) replaces the oracle's own selection by a given one (to check the stages
    after routing on exactly the assignments another implementation made); ``tokens`` (optional)
    restricts y to those token indices (y_t depends on token t alone once dispatch is fixed);
    ``expert_weights`` (optional) is a callable e -> (W_gate_e, W_up_e, W_down_e) used instead of
    indexing the full weight tensors. With ``magnitudes``, res["magnitude"] holds, per element of
    y, the sum of the absolute values of the terms the combine adds, sum_j |w_tj E_j(x_t)_i| +
    sum_s |E^s(x_t)_i|: the scale of any rounding of those terms, which y itself can undercut
    when they cancel.
    """
    x64 = _f64(x)
    T, d = x64.shape
    r = route(x64, W_r, k, b, renorm, scoring)
    E = r["g"].shape[1]
    S = r["topk_idx"] if topk_idx is None else np.asarray(topk_idx, dtype=np.int64)
    w = gate_weights(r["g"], S, renorm)
    n = expert_loads(S, E)
    C = capacity(c, k, T, E)
    dsp = dispatch(S, E, C)
    stats = balance_stats(n, r["probs"], r["lse"], k, lam)
    want = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    want_set = set(int(t) for t in want)
    # expert outputs for the kept rows of the wanted tokens only
    out_perm = {}
    for e in range(E):
        rows_e = [(int(dsp["offsets"][e]) + p, int(dsp["perm_token"][dsp["offsets"][e] + p]))
                  for p in range(int(dsp["kept"][e]))]
        rows_e = [(rr, t) for rr, t in rows_e if t in want_set]
        if not rows_e:
            continue
        We = expert_weights(e) if expert_weights is not None else (W_gate[e], W_up[e], W_down[e])
        X = x64[[t for _, t in rows_e]]
        O = swiglu_expert(X, *We)
        for i, (rr, _) in enumerate(rows_e):
            out_perm[rr] = O[i]
    y = np.zeros((len(want), d))
    xs = x64[want]
    if shared:
        y += shared_experts(xs, shared)
    for i, t in enumerate(want):
        for j in range(k):
            rr = int(dsp["row"][t, j])
            if rr >= 0:
                y[i] += w[t, j] * out_perm[rr]
    mag = None
    if magnitudes:
        mag = np.zeros((len(want), d))
        for Ws in shared:
            mag += np.abs(swiglu_expert(xs, *Ws))
        for i, t in enumerate(want):
            for j in range(k):
                rr = int(dsp["row"][t, j])
                if rr >= 0:
                    mag[i] += np.abs(w[t, j] * out_perm[rr])
    res = {"y": y, "magnitude": mag, "tokens": want, "topk_idx": S, "topk_w": w, "n": n, "C": C,
           **dsp, **stats,
           "diag": diagnostics(n, r["probs"]),
           "lse": r["lse"], "g": r["g"], "margin": r["margin"], "s": r["s"]}
    if b is not None:
        res["b_new"] = bias_update(b, n, k, T, gamma)
    return res

"""Pins of the CPU oracle against what the source pages and mathematics fix (no GPU needed).

Each test checks one oracle step against something other than the oracle itself: a closed form,
an invariant the pages' formulas imply, brute force on tiny inputs, an independent formula from a
page, or a library routine. ``test_planted_mistakes_are_caught`` plants plausible mistakes in the
oracle and checks that these pins fail on each.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import workloads
from oracle import moe_oracle as O

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")))


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ------------------------------------------------------------------------------------- softmax

def check_softmax(mod=O):
    l = _rand((64, 12), 1, 3.0)
    g, lse = mod.softmax_lse(l)
    assert np.allclose(g.sum(1), 1.0, atol=1e-14)
    # scipy's logsumexp is an independent library routine
    from scipy.special import logsumexp
    assert np.allclose(lse, logsumexp(l, axis=1), atol=1e-13, rtol=0)
    # each probability against math.exp on one row, in plain Python
    row = [float(v) for v in l[5]]
    den = sum(math.exp(v) for v in row)
    assert np.allclose(g[5], [math.exp(v) / den for v in row], rtol=1e-13)
    # zero router => uniform probabilities, lse = ln E
    g0, lse0 = mod.softmax_lse(np.zeros((3, 8)))
    assert np.allclose(g0, 1.0 / 8, rtol=1e-15, atol=0) and np.allclose(lse0, math.log(8), rtol=1e-15)
    # constant logits a => lse = a + ln E; huge logits stay finite (max subtraction)
    g1, lse1 = mod.softmax_lse(np.full((2, 5), 1000.0))
    assert np.allclose(lse1, 1000.0 + math.log(5), rtol=1e-15) and np.all(np.isfinite(g1))


def test_softmax_pins():
    check_softmax()


# --------------------------------------------------------------------------------------- top-k

def _topk_repeated_argmax(s_row, k):
    """k rounds of 'take the largest remaining score, lowest index on ties' in plain Python."""
    left = list(range(len(s_row)))
    out = []
    for _ in range(k):
        best = left[0]
        for e in left[1:]:
            if s_row[e] > s_row[best]:
                best = e
        out.append(best)
        left.remove(best)
    return out


def check_topk(mod=O):
    rng = np.random.default_rng(2)
    # scores on a coarse grid so that ties are frequent
    s = rng.integers(0, 5, size=(200, 7)).astype(np.float64) / 4.0
    for k in (1, 2, 3, 7):
        S = mod.top_k(s, k)
        for t in range(s.shape[0]):
            assert list(S[t]) == _topk_repeated_argmax(list(s[t]), k)
    # exhaustive over k-subsets on distinct scores: the top-k set maximises the score sum
    s = rng.permutation(np.arange(6 * 40, dtype=np.float64)).reshape(40, 6)
    for k in (1, 2, 3, 4):
        S = mod.top_k(s, k)
        for t in range(s.shape[0]):
            best = max(itertools.combinations(range(6), k), key=lambda c: sum(s[t, list(c)]))
            assert set(S[t]) == set(best)
            assert all(s[t, S[t, j]] > s[t, S[t, j + 1]] for j in range(k - 1))
    # library: torch.topk on distinct scores
    s = _rand((50, 16), 3)
    vals, idx = torch.topk(torch.from_numpy(s), 4, dim=1)
    assert np.array_equal(mod.top_k(s, 4), idx.numpy())


def test_topk_pins():
    check_topk()


def test_topk_margin():
    s = np.array([[0.5, 0.1, 0.3, 0.2], [0.25, 0.25, 0.25, 0.25]])
    assert np.allclose(O.topk_margin(s, 2), [0.1, 0.0])
    assert np.all(np.isinf(O.topk_margin(s, 4)))


# ---------------------------------------------------------------------------------- gates/renorm

def check_gates(mod=O):
    l = _rand((100, 10), 4, 2.0)
    g, _ = mod.softmax_lse(l)
    S = mod.top_k(g, 3)
    w = mod.gate_weights(g, S, True)
    assert np.allclose(w.sum(1), 1.0, atol=1e-14)
    # "Softmax(TopK(W_g x, k))" with the others set to -inf ([AIATTN] §2.2): an independent form
    masked = np.full_like(l, -np.inf)
    np.put_along_axis(masked, S, np.take_along_axis(l, S, 1), 1)
    ref = np.exp(masked - masked.max(1, keepdims=True))
    ref /= ref.sum(1, keepdims=True)
    assert np.allclose(w, np.take_along_axis(ref, S, 1), rtol=1e-13)
    # without renormalisation the gates are the raw probabilities
    assert np.array_equal(mod.gate_weights(g, S, False), np.take_along_axis(g, S, 1))


def test_gate_pins():
    check_gates()


# ----------------------------------------------------------------------- sigmoid scoring (V3)

def check_sigmoid(mod=O):
    l = _rand((80, 16), 11, 4.0)
    l[3, :4] = [0.0, math.log(3.0), -math.log(3.0), 60.0]
    s = mod.sigmoid_scores(l)
    # scipy's logistic function is an independent library routine
    from scipy.special import expit
    assert np.allclose(s, expit(l), rtol=1e-15, atol=0)
    # closed forms: sigma(0) = 1/2, sigma(ln 3) = 3/4, sigma(-ln 3) = 1/4; sigma(l) + sigma(-l) = 1
    assert s[3, 0] == 0.5
    assert math.isclose(s[3, 1], 0.75, rel_tol=1e-15) and math.isclose(s[3, 2], 0.25, rel_tol=1e-15)
    assert np.allclose(s + mod.sigmoid_scores(-l), 1.0, atol=1e-15)
    # no bias: sigmoid is increasing, so it picks the same experts in the same order as softmax
    g, _ = mod.softmax_lse(l)
    for k in (1, 2, 6):
        assert np.array_equal(mod.top_k(s, k), mod.top_k(g, k))
    # gates: the chosen scores renormalised; with every expert chosen they are s / sum_e s
    S = mod.top_k(s, 16)
    w = mod.gate_weights(s, S, True)
    dist = mod.score_distribution(s, "sigmoid")
    assert np.allclose(w, np.take_along_axis(dist, S, 1), rtol=1e-14)
    # zero router: every score 1/2, renormalised gates 1/k exactly
    s0 = mod.sigmoid_scores(np.zeros((10, 6)))
    assert np.all(s0 == 0.5)
    w0 = mod.gate_weights(s0, mod.top_k(s0, 4), True)
    assert np.all(w0 == 0.25)


def test_sigmoid_pins():
    check_sigmoid()


def check_sigmoid_stats(mod=O):
    T, E, k = 64, 8, 2
    l = _rand((T, E), 12, 2.0)
    r = mod.route(l, np.eye(E), k, scoring="sigmoid")  # x = l, W_r = I: logits are l itself
    assert np.allclose(r["logits"], l)
    st = mod.balance_stats(mod.expert_loads(r["topk_idx"], E), r["probs"], r["lse"], k, 0.01)
    assert abs(st["P"].sum() - 1.0) < 1e-14 and abs(st["f"].sum() - 1.0) < 1e-14
    # P_e against a plain Python mean of s_te / sum_e' s_te'
    srow = [[1.0 / (1.0 + math.exp(-float(v))) for v in row] for row in l]
    ref = sum(row[5] / sum(row) for row in srow) / T
    assert math.isclose(st["P"][5], ref, rel_tol=1e-13)
    # z is the softmax lse of the raw logits, whatever the scoring
    from scipy.special import logsumexp
    assert math.isclose(st["z"], float((logsumexp(l, axis=1) ** 2).mean()), rel_tol=1e-13)
    # zero router: uniform scores => aux = lambda exactly
    r0 = mod.route(np.zeros((T, E)), np.eye(E), k, scoring="sigmoid")
    st0 = mod.balance_stats(mod.expert_loads(r0["topk_idx"], E), r0["probs"], r0["lse"], k,
                            GOLDEN["uniform_router_aux"]["lambda"])
    assert math.isclose(st0["aux"], GOLDEN["uniform_router_aux"]["aux"], rel_tol=1e-14)


def test_sigmoid_stats_pins():
    check_sigmoid_stats()


def test_sigmoid_bias_changes_selection_not_gates():
    # ALF-LB with sigmoid scores: a large bias on expert 0 forces it into every selection, while
    # each chosen gate stays the unbiased score renormalised over the chosen set
    T, E, k = 30, 6, 2
    l = _rand((T, E), 13)
    b = np.zeros(E)
    b[0] = 5.0
    r = O.route(l, np.eye(E), k, b=b, scoring="sigmoid")
    assert np.all(r["topk_idx"][:, 0] == 0)
    s = O.sigmoid_scores(l)
    sel = np.take_along_axis(s, r["topk_idx"], 1)
    assert np.allclose(r["topk_w"], sel / sel.sum(1, keepdims=True), rtol=1e-14)


def test_sigmoid_layer_matches_softmax_when_selection_agrees():
    # no bias and k = 1: both scorings pick the argmax and the renormalised gate is 1, so the whole
    # layer output is identical
    x, W_r, Wg, Wu, Wd = _tiny_layer(k=1)
    a = O.layer_forward(x, W_r, Wg, Wu, Wd, 1, scoring="softmax")
    bb = O.layer_forward(x, W_r, Wg, Wu, Wd, 1, scoring="sigmoid")
    assert np.array_equal(a["topk_idx"], bb["topk_idx"])
    assert np.allclose(a["y"], bb["y"], rtol=1e-13, atol=1e-13)
    assert np.array_equal(a["n"], bb["n"]) and math.isclose(a["z"], bb["z"], rel_tol=1e-15)


# --------------------------------------------------------------------------------- statistics

def check_stats(mod=O):
    T, E, lam = 96, 6, 0.01
    l = _rand((T, E), 5)
    g, lse = mod.softmax_lse(l)
    for k in (1, 2, 3):
        S = mod.top_k(g, k)
        n = mod.expert_loads(S, E)
        st = mod.balance_stats(n, g, lse, k, lam)
        assert abs(st["f"].sum() - 1.0) < 1e-14 and abs(st["P"].sum() - 1.0) < 1e-14
        assert n.sum() == k * T
        if k == 1:  # the argmax-fraction form of [AIATTN] §4.2.1 and [CMP] §2.1
            am = np.argmax(g, axis=1)
            assert np.allclose(st["f"], [(am == e).mean() for e in range(E)])
        # P_e against a plain Python mean of the column
        assert math.isclose(st["P"][2], sum(float(v) for v in g[:, 2]) / T, rel_tol=1e-13)
    # zero router: P uniform => aux = lambda exactly; z = (ln E)^2
    g0, lse0 = mod.softmax_lse(np.zeros((40, 8)))
    S0 = mod.top_k(g0, 2)
    st0 = mod.balance_stats(mod.expert_loads(S0, 8), g0, lse0, 2, GOLDEN["uniform_router_aux"]["lambda"])
    assert math.isclose(st0["aux"], GOLDEN["uniform_router_aux"]["aux"], rel_tol=1e-14)
    assert math.isclose(st0["z"], GOLDEN["uniform_router_z"]["z"], rel_tol=1e-14)
    # uniform loads by construction (token t prefers experts t%E and (t+1)%E) => aux = lambda
    T2, E2, k2 = 48, 6, 2
    l2 = np.zeros((T2, E2))
    for t in range(T2):
        l2[t, t % E2] = 3.0 + 0.1 * (t % 5)
        l2[t, (t + 1) % E2] = 2.0
    g2, lse2 = mod.softmax_lse(l2)
    S2 = mod.top_k(g2, k2)
    n2 = mod.expert_loads(S2, E2)
    assert np.all(n2 == k2 * T2 // E2)
    st2 = mod.balance_stats(n2, g2, lse2, k2, 0.01)
    assert math.isclose(st2["aux"], 0.01, rel_tol=1e-14)


def test_stats_pins():
    check_stats()


# ---------------------------------------------------------------------------------- diagnostics

def check_diagnostics(mod=O):
    E = 8
    # entropy: uniform probabilities give ln E, one-hot rows give 0; scipy's entropy (natural log)
    assert math.isclose(mod.routing_entropy(np.full((5, E), 1.0 / E)), math.log(E), rel_tol=1e-14)
    assert mod.routing_entropy(np.eye(E)) == 0.0
    from scipy.stats import entropy
    g, _ = mod.softmax_lse(_rand((50, E), 21, 2.0))
    assert math.isclose(mod.routing_entropy(g), float(np.mean([entropy(r) for r in g])), rel_tol=1e-13)
    # Gini: equal loads 0; one expert with everything (E-1)/E; the sorted closed form
    # G = 2 sum_i i x_(i) / (E sum x) - (E + 1) / E  (x ascending, i = 1..E)
    assert mod.load_gini(np.full(E, 7)) == 0.0
    assert math.isclose(mod.load_gini(np.array([0] * (E - 1) + [40])), (E - 1) / E, rel_tol=1e-14)
    x = np.array([3, 9, 0, 14, 5, 5, 1, 27])
    xs = np.sort(x)
    ref = 2.0 * sum((i + 1) * v for i, v in enumerate(xs)) / (E * xs.sum()) - (E + 1) / E
    assert math.isclose(mod.load_gini(x), ref, rel_tol=1e-13)
    # max/mean load
    assert math.isclose(mod.load_max_over_mean(x), 27 / (x.sum() / E), rel_tol=1e-14)
    assert mod.load_max_over_mean(np.full(E, 3)) == 1.0
    # importance CV^2: equal importance 0; two experts (a, b) give ((a - b) / (a + b))^2
    assert mod.importance_cv2(np.full(E, 2.5)) == 0.0
    assert math.isclose(mod.importance_cv2(np.array([3.0, 1.0])), 0.25, rel_tol=1e-14)


def test_diagnostics_pins():
    check_diagnostics()


# ----------------------------------------------------------------------------- expert choice

def check_expert_choice(mod=O):
    T, E, r = 50, 6, 7
    l = _rand((T, E), 31, 2.0)
    ch = mod.expert_choice(l, r)
    assert ch.shape == (E, r)
    for e in range(E):
        assert np.all(np.diff(ch[e]) > 0)  # ascending, distinct
        # torch.topk on distinct values is an independent library routine
        ref = torch.topk(torch.from_numpy(l[:, e]), r).indices.numpy()
        assert set(ch[e].tolist()) == set(ref.tolist())
    # characterisation with ties: t is taken iff fewer than r tokens beat it (larger score, or
    # equal score and lower index); integer scores make many ties
    li = np.random.default_rng(32).integers(0, 4, size=(20, 3)).astype(np.float64)
    ch2 = mod.expert_choice(li, 5)
    for e in range(3):
        for t in range(20):
            beat = sum(1 for u in range(20) if li[u, e] > li[t, e] or (li[u, e] == li[t, e] and u < t))
            assert (t in set(ch2[e].tolist())) == (beat < 5)
    # all scores equal: the first r tokens
    assert np.array_equal(mod.expert_choice(np.zeros((9, 2)), 4), [[0, 1, 2, 3]] * 2)
    # r = ceil(c k T / E), c <= 0 read as 1, at most T
    assert mod.expert_choice_capacity(1.0, 2, 10, 3) == GOLDEN["capacity_ceil"]["C"]
    assert mod.expert_choice_capacity(None, 2, 10, 3) == 7 and mod.expert_choice_capacity(0.0, 2, 10, 3) == 7
    assert mod.expert_choice_capacity(8.0, 2, 10, 3) == 10


def test_expert_choice_pins():
    check_expert_choice()


def test_expert_choice_layer_pins():
    x, W_r, Wg, Wu, Wd = _tiny_layer(T=30, E=4, k=2)
    T, E = 30, 4
    # r = T: every expert takes every token; renormalised gates are the softmax itself, so y is the
    # dense soft mixture sum_e g_te E_e(x_t), computed here without any selection
    res = O.layer_forward_expert_choice(x, W_r, Wg, Wu, Wd, 2, c=E / 2.0)
    assert res["r"] == T and res["uncovered"] == 0
    from scipy.special import softmax
    g = softmax(x @ W_r.T, axis=1)
    dense = sum(g[:, e:e + 1] * O.swiglu_expert(x, Wg[e], Wu[e], Wd[e]) for e in range(E))
    assert np.allclose(res["y"], dense, rtol=1e-12, atol=1e-12)
    # identical experts + renorm: every covered token gets FFN(x); uncovered tokens get 0
    Wg1, Wu1, Wd1 = (np.repeat(W[:1], E, axis=0) for W in (Wg, Wu, Wd))
    res2 = O.layer_forward_expert_choice(x, W_r, Wg1, Wu1, Wd1, 1, c=0.5)
    ffn = O.swiglu_expert(x, Wg1[0], Wu1[0], Wd1[0])
    covered = np.zeros(T, dtype=bool)
    for e in range(E):
        covered[res2["chosen"][e]] = True
    assert res2["uncovered"] == int((~covered).sum()) > 0
    assert np.allclose(res2["y"][covered], ffn[covered], rtol=1e-12, atol=1e-12)
    assert np.all(res2["y"][~covered] == 0.0)
    # equal loads: f = 1/E, Gini 0, max/mean 1
    assert np.allclose(res2["f"], 1.0 / E) and res2["diag"]["gini"] == 0.0
    assert res2["diag"]["max_over_mean"] == 1.0


# -------------------------------------------------------------------------- loss backward

def _balance_loss(mod, l, f, lam, zc, scoring):
    # L = aux + zc z evaluated from its forward definitions (f held fixed)
    l = np.asarray(l, dtype=np.float64)
    g, lse = mod.softmax_lse(l)
    p = g if scoring == "softmax" else mod.score_distribution(mod.sigmoid_scores(l), "sigmoid")
    T, E = l.shape
    aux = lam * E * float((f * p.sum(axis=0) / T).sum())
    return aux + zc * float((lse ** 2).mean())


def check_loss_backward(mod=O):
    T, E = 9, 5
    l = _rand((T, E), 41, 1.5)
    f = np.array([0.3, 0.1, 0.25, 0.05, 0.3])
    lam, zc = 0.37, 0.8
    for scoring in ("softmax", "sigmoid"):
        dl = mod.balance_loss_grad_logits(l, f, lam, zc, scoring)
        # central finite differences of the forward loss
        h = 1e-6
        fd = np.zeros_like(l)
        for t in range(T):
            for e in range(E):
                lp, lm = l.copy(), l.copy()
                lp[t, e] += h
                lm[t, e] -= h
                fd[t, e] = (_balance_loss(mod, lp, f, lam, zc, scoring) -
                            _balance_loss(mod, lm, f, lam, zc, scoring)) / (2 * h)
        assert np.allclose(dl, fd, rtol=1e-6, atol=1e-9), scoring
        # torch autograd in float64 on the same loss written with torch ops
        lt = torch.tensor(l, requires_grad=True)
        ft = torch.tensor(f)
        if scoring == "softmax":
            p = torch.softmax(lt, dim=1)
        else:
            sg = torch.sigmoid(lt)
            p = sg / sg.sum(dim=1, keepdim=True)
        L = lam * E * (ft * p.mean(dim=0)).sum() + zc * (torch.logsumexp(lt, dim=1) ** 2).mean()
        L.backward()
        assert np.allclose(dl, lt.grad.numpy(), rtol=1e-12, atol=1e-15), scoring
    # zero router and equal f: the aux term has zero gradient (uniform P is stationary)
    dl0 = mod.balance_loss_grad_logits(np.zeros((4, E)), np.full(E, 1.0 / E), 1.0, 0.0)
    assert np.allclose(dl0, 0.0, atol=1e-15)
    # the chain through the router: dW_r = dl^T x and dx = dl W_r, against autograd
    x = _rand((T, 6), 42)
    W = _rand((E, 6), 43, 0.4)
    out = mod.balance_loss_backward(x, W, f, lam, zc)
    xt = torch.tensor(x, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    lt = xt @ Wt.T
    L = lam * E * (torch.tensor(f) * torch.softmax(lt, 1).mean(0)).sum() + zc * (torch.logsumexp(lt, 1) ** 2).mean()
    L.backward()
    assert np.allclose(out["dW_r"], Wt.grad.numpy(), rtol=1e-12, atol=1e-15)
    assert np.allclose(out["dx"], xt.grad.numpy(), rtol=1e-12, atol=1e-15)


def test_loss_backward_pins():
    check_loss_backward()


# ---------------------------------------------------------------------------- layer backward

def _torch_layer_loss(x, Wr, Wg, Wu, Wd, dy, S, kept, f, k, renorm, lam, zc, scoring, shared):
    # the layer written densely with torch ops: every expert on every token, masked by the fixed
    # selection and capacity; L = <dy, y> + aux + zc z with f fixed
    l = x @ Wr.T
    if scoring == "softmax":
        g = torch.softmax(l, dim=1)
        p = g
    else:
        g = torch.sigmoid(l)
        p = g / g.sum(dim=1, keepdim=True)
    T, E = g.shape
    mask = torch.zeros(T, E, dtype=torch.float64)
    for t in range(T):
        for j in range(k):
            if kept[t, j]:
                mask[t, S[t, j]] = 1.0
    sel = torch.zeros(T, E, dtype=torch.float64)
    for t in range(T):
        for j in range(k):
            sel[t, S[t, j]] = 1.0
    gw = g * sel
    w = gw / gw.sum(dim=1, keepdim=True) if renorm else gw
    y = torch.zeros_like(x)
    for e in range(E):
        h = torch.nn.functional.silu(x @ Wg[e].T) * (x @ Wu[e].T)
        y = y + (w[:, e] * mask[:, e])[:, None] * (h @ Wd[e].T)
    for sg, su, sd in shared:
        y = y + (torch.nn.functional.silu(x @ sg.T) * (x @ su.T)) @ sd.T
    aux = lam * E * (f * p.mean(dim=0)).sum()
    z = (torch.logsumexp(l, dim=1) ** 2).mean()
    return (dy * y).sum() + aux + zc * z


def check_layer_backward(mod=O):
    T, d, E, k, M = 14, 6, 4, 2, 5
    rng = np.random.default_rng(51)
    x = rng.standard_normal((T, d))
    Wr = rng.standard_normal((E, d)) * 0.5
    Wg = rng.standard_normal((E, M, d)) * 0.4
    Wu = rng.standard_normal((E, M, d)) * 0.4
    Wd = rng.standard_normal((E, d, M)) * 0.4
    dy = rng.standard_normal((T, d))
    sh = [tuple(rng.standard_normal(sz) * 0.4 for sz in ((M, d), (M, d), (d, M)))]
    for scoring, renorm, c, shared in (("softmax", True, None, ()), ("sigmoid", False, 0.75, sh),
                                       ("softmax", True, 0.6, sh)):
        ref = mod.layer_backward(x, Wr, Wg, Wu, Wd, dy, k, shared=shared, c=c, renorm=renorm,
                                 lam=0.3, z_coef=0.7, scoring=scoring)
        fw = O.layer_forward(x, Wr, Wg, Wu, Wd, k, c=c, renorm=renorm, scoring=scoring)
        S = fw["topk_idx"]
        kept = fw["row"] >= 0
        f = torch.tensor(fw["n"] / float(k * T))
        ts = [torch.tensor(a, requires_grad=True) for a in (x, Wr, Wg, Wu, Wd)]
        tsh = [tuple(torch.tensor(a, requires_grad=True) for a in s_) for s_ in shared]
        L = _torch_layer_loss(*ts, torch.tensor(dy), S, kept, f, k, renorm, 0.3, 0.7, scoring, tsh)
        L.backward()
        for name, t_ in zip(("dx", "dW_r", "dW_gate", "dW_up", "dW_down"), ts):
            assert np.allclose(ref[name], t_.grad.numpy(), rtol=1e-10, atol=1e-12), (scoring, name)
        for (a, b_, c_), (tg, tu, td) in zip(ref["shared"], tsh):
            assert np.allclose(a, tg.grad.numpy(), rtol=1e-10, atol=1e-12)
            assert np.allclose(b_, tu.grad.numpy(), rtol=1e-10, atol=1e-12)
            assert np.allclose(c_, td.grad.numpy(), rtol=1e-10, atol=1e-12)
    # SiLU' against a central difference
    zz = np.linspace(-6, 6, 25)
    fd = (O.silu(zz + 1e-6) - O.silu(zz - 1e-6)) / 2e-6
    assert np.allclose(mod.silu_grad(zz), fd, rtol=1e-7, atol=1e-9)


def test_layer_backward_pins():
    check_layer_backward()


def _torch_layer_loss_ec(x, Wr, Wg, Wu, Wd, dy, member, f, renorm, lam, zc, scoring, shared):
    # the expert-choice layer written densely: every expert on every token, masked by the fixed
    # membership; gates renormalised over the experts that took the token
    l = x @ Wr.T
    if scoring == "softmax":
        g = torch.softmax(l, dim=1)
        p = g
    else:
        g = torch.sigmoid(l)
        p = g / g.sum(dim=1, keepdim=True)
    gm = g * member
    if renorm:
        den = gm.sum(dim=1, keepdim=True)
        w = torch.where(den > 0, gm / torch.where(den > 0, den, torch.ones_like(den)), gm)
    else:
        w = gm
    y = torch.zeros_like(x)
    for e in range(g.shape[1]):
        h = torch.nn.functional.silu(x @ Wg[e].T) * (x @ Wu[e].T)
        y = y + w[:, e:e + 1] * (h @ Wd[e].T)
    for sg, su, sd in shared:
        y = y + (torch.nn.functional.silu(x @ sg.T) * (x @ su.T)) @ sd.T
    aux = lam * g.shape[1] * (f * p.mean(dim=0)).sum()
    z = (torch.logsumexp(l, dim=1) ** 2).mean()
    return (dy * y).sum() + aux + zc * z


def check_layer_backward_ec(mod=O):
    T, d, E, k, M = 13, 6, 4, 1, 5
    rng = np.random.default_rng(61)
    x = rng.standard_normal((T, d))
    Wr = rng.standard_normal((E, d)) * 0.5
    Wg = rng.standard_normal((E, M, d)) * 0.4
    Wu = rng.standard_normal((E, M, d)) * 0.4
    Wd = rng.standard_normal((E, d, M)) * 0.4
    dy = rng.standard_normal((T, d))
    sh = [tuple(rng.standard_normal(sz) * 0.4 for sz in ((M, d), (M, d), (d, M)))]
    for scoring, renorm, c, shared in (("softmax", True, None, ()), ("sigmoid", False, 1.5, sh),
                                       ("softmax", True, 0.6, sh)):
        ref = mod.layer_backward_expert_choice(x, Wr, Wg, Wu, Wd, dy, k, shared=shared, c=c,
                                               renorm=renorm, lam=0.3, z_coef=0.7, scoring=scoring)
        fw = O.layer_forward_expert_choice(x, Wr, Wg, Wu, Wd, k, c=c, renorm=renorm,
                                           scoring=scoring)
        member = np.zeros((T, E))
        for e in range(E):
            member[fw["chosen"][e], e] = 1.0
        assert (member.sum(axis=1) == 0).any() or c is None or c > 1  # some token uncovered
        ts = [torch.tensor(a, requires_grad=True) for a in (x, Wr, Wg, Wu, Wd)]
        tsh = [tuple(torch.tensor(a, requires_grad=True) for a in s_) for s_ in shared]
        L = _torch_layer_loss_ec(*ts, torch.tensor(dy), torch.tensor(member),
                                 torch.tensor(fw["f"]), renorm, 0.3, 0.7, scoring, tsh)
        L.backward()
        for name, t_ in zip(("dx", "dW_r", "dW_gate", "dW_up", "dW_down"), ts):
            assert np.allclose(ref[name], t_.grad.numpy(), rtol=1e-10, atol=1e-12), (scoring, name)
        for (a, b_, c_), (tg, tu, td) in zip(ref["shared"], tsh):
            assert np.allclose(a, tg.grad.numpy(), rtol=1e-10, atol=1e-12)
            assert np.allclose(b_, tu.grad.numpy(), rtol=1e-10, atol=1e-12)
            assert np.allclose(c_, td.grad.numpy(), rtol=1e-10, atol=1e-12)
        mref = mod.layer_backward_expert_choice(x, Wr, Wg, Wu, Wd, dy, k, shared=shared, c=c,
                                                renorm=renorm, lam=0.3, z_coef=0.7,
                                                scoring=scoring, magnitudes=True)["magnitude"]
        for key in ("dx", "dW_r", "dW_gate", "dW_up", "dW_down"):
            assert (mref[key] >= np.abs(ref[key]) * (1 - 1e-12)).all(), key


def test_layer_backward_expert_choice_pins():
    check_layer_backward_ec()


def test_layer_backward_sampled_matches_whole():
    # the per-entry evaluation agrees with the whole backward on every token and every column,
    # with capacity drops, shared experts, sigmoid scores and a bias
    T, d, E, k, M = 16, 6, 4, 2, 5
    rng = np.random.default_rng(91)
    args = (rng.standard_normal((T, d)), rng.standard_normal((E, d)) * 0.5,
            rng.standard_normal((E, M, d)) * 0.4, rng.standard_normal((E, M, d)) * 0.4,
            rng.standard_normal((E, d, M)) * 0.4, rng.standard_normal((T, d)))
    sh = [tuple(rng.standard_normal(sz) * 0.4 for sz in ((M, d), (M, d), (d, M))) for _ in range(2)]
    bias = rng.uniform(-0.1, 0.1, E)
    for scoring, renorm, c, b in (("softmax", True, 0.7, None), ("sigmoid", False, None, bias)):
        kw = dict(b=b, shared=sh, c=c, renorm=renorm, lam=0.2, z_coef=0.5, scoring=scoring)
        whole = O.layer_backward(*args, k, magnitudes=True, **kw)
        cols = [(e, m) for e in range(E) for m in range(M)]
        part = O.layer_backward_sampled(*args, k, tokens=range(T), expert_cols=cols,
                                        shared_cols=range(2 * M), **kw)
        assert np.allclose(part["dx"], whole["dx"], rtol=1e-12, atol=1e-13)
        assert np.allclose(part["magnitude"]["dx"], whole["magnitude"]["dx"], rtol=1e-12)
        for i, (e, m) in enumerate(cols):
            for key, ref, mref in (("dW_gate", whole["dW_gate"][e, m], whole["magnitude"]["dW_gate"][e, m]),
                                   ("dW_up", whole["dW_up"][e, m], whole["magnitude"]["dW_up"][e, m]),
                                   ("dW_down", whole["dW_down"][e][:, m], whole["magnitude"]["dW_down"][e][:, m])):
                assert np.allclose(part[key][i], ref, rtol=1e-12, atol=1e-13), (key, e, m)
                assert np.allclose(part["magnitude"][key][i], mref, rtol=1e-12), (key, e, m)
        sg = np.concatenate([t[0] for t in whole["shared"]], 0)
        su = np.concatenate([t[1] for t in whole["shared"]], 0)
        sd = np.concatenate([t[2] for t in whole["shared"]], 1)
        for m in range(2 * M):
            assert np.allclose(part["dWs_gate"][m], sg[m], rtol=1e-12, atol=1e-13)
            assert np.allclose(part["dWs_up"][m], su[m], rtol=1e-12, atol=1e-13)
            assert np.allclose(part["dWs_down"][m], sd[:, m], rtol=1e-12, atol=1e-13)


def test_layer_backward_magnitudes_dominate():
    # the rounding-bound scales: same gradients with or without them, and each scale is at least
    # the absolute value of its gradient (a sum is bounded by the sum of its terms' magnitudes)
    T, d, E, k, M = 12, 5, 3, 2, 4
    rng = np.random.default_rng(77)
    args = (rng.standard_normal((T, d)), rng.standard_normal((E, d)) * 0.5,
            rng.standard_normal((E, M, d)) * 0.4, rng.standard_normal((E, M, d)) * 0.4,
            rng.standard_normal((E, d, M)) * 0.4, rng.standard_normal((T, d)))
    sh = [tuple(rng.standard_normal(sz) * 0.4 for sz in ((M, d), (M, d), (d, M)))]
    a = O.layer_backward(*args, k, shared=sh, c=0.8, lam=0.2, z_coef=0.5)
    b = O.layer_backward(*args, k, shared=sh, c=0.8, lam=0.2, z_coef=0.5, magnitudes=True)
    mag = b["magnitude"]
    for key in ("dx", "dW_r", "dW_gate", "dW_up", "dW_down"):
        assert np.array_equal(a[key], b[key])
        assert (mag[key] >= np.abs(b[key]) * (1 - 1e-12)).all(), key
        assert mag[key].max() > 0
    for grads, mags in zip(b["shared"], mag["shared"]):
        for g_, m_ in zip(grads, mags):
            assert (m_ >= np.abs(g_) * (1 - 1e-12)).all()


# ----------------------------------------------------------------------------- capacity/dispatch

def test_capacity_closed_forms():
    c = GOLDEN["capacity_skewed"]
    assert O.capacity(c["c"], c["k"], c["T"], c["E"]) == c["C"]
    c = GOLDEN["capacity_ceil"]
    assert O.capacity(c["c"], c["k"], c["T"], c["E"]) == c["C"]
    assert O.capacity(None, 2, 10, 3) is None and O.capacity(0.0, 2, 10, 3) is None
    # c is the float32 the caller passes: fp32(0.05) is just above 0.05, so 0.05*2*40/4 rounds up to 2
    assert O.capacity(0.05, 2, 40, 4) == 2 and O.capacity(0.03125, 2, 40, 4) == 1
    cfg = workloads.CONFIGS["skewed_capacity"]
    assert O.capacity(cfg.c, cfg.k, cfg.T, cfg.E) == GOLDEN["capacity_skewed"]["C"]


def _counter_simulation(S, E, C):
    """Sequential first-come-first-kept: walk tokens ascending, one counter per expert."""
    T, k = S.shape
    cnt = [0] * E
    keep = np.zeros((T, k), dtype=bool)
    for t in range(T):
        for j in range(k):
            e = int(S[t, j])
            cnt[e] += 1
            keep[t, j] = C is None or cnt[e] <= C
    return keep, np.array(cnt)


def _check_dispatch_against_simulation(mod, S, E, C):
    dsp = mod.dispatch(S, E, C)
    keep, n = _counter_simulation(S, E, C)
    assert np.array_equal(dsp["row"] >= 0, keep)
    assert np.array_equal(dsp["kept"] + dsp["overflow"], n)
    assert dsp["kept"].sum() + dsp["overflow"].sum() == S.size
    if C is not None:
        assert np.all(dsp["kept"] <= C)
        assert np.all(dsp["overflow"][n <= C] == 0)
    # perm_token is a bijection onto the kept assignments, ascending tokens within a segment
    rows = dsp["row"][keep]
    assert sorted(rows.tolist()) == list(range(int(dsp["offsets"][-1])))
    for e in range(E):
        seg = dsp["perm_token"][dsp["offsets"][e]:dsp["offsets"][e + 1]]
        assert np.all(np.diff(seg) > 0)
        assert np.all([e in S[t] for t in seg])
    for t in range(S.shape[0]):
        for j in range(S.shape[1]):
            if keep[t, j]:
                r = dsp["row"][t, j]
                assert dsp["perm_token"][r] == t
                assert dsp["offsets"][S[t, j]] <= r < dsp["offsets"][S[t, j] + 1]


def check_dispatch(mod=O, exhaustive=True):
    T, E, k = 5, 4, 2
    subsets = list(itertools.combinations(range(E), k))
    cases = itertools.product(subsets, repeat=T) if exhaustive else \
        [tuple(subsets[i] for i in np.random.default_rng(s).integers(0, len(subsets), T)) for s in range(200)]
    for assign in cases:
        S = np.array(assign, dtype=np.int64)
        for C in (1, 2, None):
            _check_dispatch_against_simulation(mod, S, E, C)
    # a larger random case with slot order not sorted by index
    rng = np.random.default_rng(7)
    S = np.stack([rng.permutation(9)[:3] for _ in range(300)])
    for C in (50, 100, 120, None):
        _check_dispatch_against_simulation(mod, S, 9, C)


def test_dispatch_exhaustive_tiny():
    check_dispatch(exhaustive=True)


# ------------------------------------------------------------------------------------- experts

def check_experts(mod=O):
    d = 6
    rng = np.random.default_rng(8)
    p1, p2, p3 = rng.permutation(d), rng.permutation(d), rng.permutation(d)
    Pg, Pu, Pd = np.eye(d)[p1], np.eye(d)[p2], np.eye(d)[p3]   # (P x)_i = x[p[i]]
    X = rng.standard_normal((4, d))
    out = mod.swiglu_expert(X, Pg, Pu, Pd)
    for r in range(4):
        h = [X[r, p1[i]] / (1.0 + math.exp(-X[r, p1[i]])) * X[r, p2[i]] for i in range(d)]
        assert np.allclose(out[r], [h[p3[i]] for i in range(d)], rtol=1e-14)
    # SiLU closed values
    assert mod.silu(np.array([0.0]))[0] == 0.0
    assert math.isclose(mod.silu(np.array([50.0]))[0], 50.0, rel_tol=1e-15)
    assert abs(mod.silu(np.array([-50.0]))[0]) < 1e-19
    # zero gate projection => zero output
    assert np.all(mod.swiglu_expert(X, np.zeros((3, d)), rng.standard_normal((3, d)),
                                    rng.standard_normal((d, 3))) == 0.0)


def test_expert_pins():
    check_experts()


def _tiny_layer(T=40, d=16, E=4, k=2, M=24, seed=0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    Wr = rng.standard_normal((E, d)) / math.sqrt(d)
    Wg = rng.standard_normal((E, M, d)) / math.sqrt(d)
    Wu = rng.standard_normal((E, M, d)) / math.sqrt(d)
    Wd = rng.standard_normal((E, d, M)) / math.sqrt(M)
    return x, Wr, Wg, Wu, Wd


def check_layer(mod=O):
    # E = 1, k = 1 collapses to the dense SwiGLU FFN
    x, Wr, Wg, Wu, Wd = _tiny_layer(E=1)
    res = mod.layer_forward(x, Wr, Wg, Wu, Wd, k=1)
    assert np.allclose(res["y"], mod.swiglu_expert(x, Wg[0], Wu[0], Wd[0]), rtol=1e-13, atol=1e-14)
    # identical experts + renorm + no drops => y = FFN(x) whatever the routing
    x, Wr, Wg, Wu, Wd = _tiny_layer(E=5, k=3)
    Wg[:], Wu[:], Wd[:] = Wg[0], Wu[0], Wd[0]
    res = mod.layer_forward(x, Wr, Wg, Wu, Wd, k=3)
    assert np.allclose(res["y"], mod.swiglu_expert(x, Wg[0], Wu[0], Wd[0]), rtol=1e-12, atol=1e-13)
    # two shared experts of width M equal one of width 2M
    x, Wr, Wg, Wu, Wd = _tiny_layer()
    rng = np.random.default_rng(11)
    sh = [(rng.standard_normal((8, 16)), rng.standard_normal((8, 16)), rng.standard_normal((16, 8)))
          for _ in range(2)]
    fused = (np.concatenate([s[0] for s in sh]), np.concatenate([s[1] for s in sh]),
             np.concatenate([s[2] for s in sh], axis=1))
    a = mod.layer_forward(x, Wr, Wg, Wu, Wd, k=2, shared=sh)
    b = mod.layer_forward(x, Wr, Wg, Wu, Wd, k=2, shared=[fused])
    assert np.allclose(a["y"], b["y"], rtol=1e-12, atol=1e-13)
    # capacity 1 on 40 tokens drops most slots; a token whose slots are all dropped gets shared only
    res = mod.layer_forward(x, Wr, Wg, Wu, Wd, k=2, shared=sh, c=1.0 / 32)  # C = ceil(0.625) = 1
    assert res["C"] == 1 and res["kept"].sum() <= 4
    none_kept = np.where((res["row"] < 0).all(1))[0]
    assert len(none_kept) > 0
    assert np.allclose(res["y"][none_kept], mod.shared_experts(x[none_kept], sh), rtol=1e-13)
    # the token subset gives the same rows as the full pass
    sub = mod.layer_forward(x, Wr, Wg, Wu, Wd, k=2, shared=sh, tokens=[3, 17, 39])
    full = mod.layer_forward(x, Wr, Wg, Wu, Wd, k=2, shared=sh)
    assert np.allclose(sub["y"], full["y"][[3, 17, 39]], rtol=1e-14, atol=0)
    # term magnitudes: never below |y| (triangle inequality), equal to it without cancellation
    full = mod.layer_forward(x, Wr, Wg, Wu, Wd, k=2, shared=sh, magnitudes=True)
    assert np.all(full["magnitude"] >= np.abs(full["y"]) * (1 - 1e-14))
    assert (full["magnitude"] > np.abs(full["y"]) * (1 + 1e-6)).any()
    x1, Wr1, Wg1, Wu1, Wd1 = _tiny_layer(E=1)
    one = mod.layer_forward(x1, Wr1, Wg1, Wu1, Wd1, k=1, magnitudes=True)
    assert np.allclose(one["magnitude"], np.abs(one["y"]), rtol=1e-14, atol=0)
    # identical experts with renormalised gates: sum_j w_j |FFN| = |FFN|
    x, Wr, Wg, Wu, Wd = _tiny_layer(E=5, k=3)
    Wg[:], Wu[:], Wd[:] = Wg[0], Wu[0], Wd[0]
    same = mod.layer_forward(x, Wr, Wg, Wu, Wd, k=3, magnitudes=True)
    assert np.allclose(same["magnitude"], np.abs(mod.swiglu_expert(x, Wg[0], Wu[0], Wd[0])),
                       rtol=1e-12, atol=1e-14)


def test_layer_pins():
    check_layer()


# ------------------------------------------------------------------- combine and shared experts

def check_combine(mod=O):
    """combine ("MoE：条件计算与路由" §7 eq. (3)) against a sparse-matrix product built by scipy,
    and against the inline combine of layer_forward."""
    import scipy.sparse as sp
    rng = np.random.default_rng(21)
    T, k, R = 30, 3, 100
    # distinct rows per slot, about a fifth dropped (-1)
    row = rng.permutation(R)[: T * k].reshape(T, k).astype(np.int64)
    row[rng.random((T, k)) < 0.2] = -1
    w = rng.random((T, k)) + 0.1
    keep = row >= 0
    tt, jj = np.nonzero(keep)
    # one-hot expert outputs (out_perm = I_R): y is the T x R gate matrix W[t, row_tj] = w_tj
    Wmat = sp.coo_matrix((w[tt, jj], (tt, row[tt, jj])), shape=(T, R)).toarray()
    y = mod.combine(T, R, row, w, np.eye(R))
    assert np.array_equal(y, Wmat)
    # general outputs: y = W out_perm (+ shared), by the sparse product
    out = rng.standard_normal((R, 9))
    sh = rng.standard_normal((T, 9))
    Ws = sp.csr_matrix((w[tt, jj], (tt, row[tt, jj])), shape=(T, R))
    assert np.allclose(mod.combine(T, 9, row, w, out), Ws @ out, rtol=1e-14, atol=1e-15)
    assert np.allclose(mod.combine(T, 9, row, w, out, sh), Ws @ out + sh, rtol=1e-14, atol=1e-15)
    # a token with every slot dropped gets exactly the shared term (0 without it)
    row[4] = -1
    assert np.all(mod.combine(T, 9, row, w, out)[4] == 0.0)
    assert np.array_equal(mod.combine(T, 9, row, w, out, sh)[4], sh[4])
    # the layer's own combine: out_perm from the dispatch rows, against layer_forward's y
    x, Wr, Wg, Wu, Wd = _tiny_layer(T=40, E=4, k=2)
    shs = [(rng.standard_normal((8, 16)), rng.standard_normal((8, 16)), rng.standard_normal((16, 8)))]
    res = mod.layer_forward(x, Wr, Wg, Wu, Wd, k=2, shared=shs, c=0.5)   # C = 5: drops
    assert res["overflow"].sum() > 0
    P = int(res["offsets"][-1])
    out_perm = np.zeros((P, 16))
    for e in range(4):
        lo, hi = int(res["offsets"][e]), int(res["offsets"][e + 1])
        out_perm[lo:hi] = O.swiglu_expert(x[res["perm_token"][lo:hi]], Wg[e], Wu[e], Wd[e])
    y2 = mod.combine(40, 16, res["row"], res["topk_w"], out_perm,
                     O.swiglu_expert(x, *shs[0]))
    assert np.allclose(y2, res["y"], rtol=1e-13, atol=1e-14)


def test_combine_pins():
    check_combine()


def check_shared(mod=O):
    """Shared experts ("MOE大模型对比篇" §3.3; the DeepseekV3MoE listing of the adg.csdn.net notes
    page, §四, adds shared_experts(identity) to the routed output): weight 1, every token."""
    rng = np.random.default_rng(23)
    x, Wr, Wg, Wu, Wd = _tiny_layer(T=24, E=4, k=2)
    sh = (rng.standard_normal((8, 16)), rng.standard_normal((8, 16)), rng.standard_normal((16, 8)))
    ffn = O.swiglu_expert(x, *sh)                 # pinned on its own (check_experts)
    zero_down = np.zeros_like(Wd)                 # every routed expert outputs 0
    res = mod.layer_forward(x, Wr, Wg, Wu, zero_down, k=2, shared=[sh], magnitudes=True)
    assert np.allclose(res["y"], ffn, rtol=1e-13, atol=1e-14)
    assert np.allclose(res["magnitude"], np.abs(ffn), rtol=1e-13, atol=1e-14)
    # S identical shared experts give S times the FFN
    res3 = mod.layer_forward(x, Wr, Wg, Wu, zero_down, k=2, shared=[sh, sh, sh])
    assert np.allclose(res3["y"], 3.0 * ffn, rtol=1e-13, atol=1e-13)
    assert np.allclose(mod.shared_experts(x, [sh]), ffn, rtol=1e-14, atol=0)
    assert np.all(mod.shared_experts(x, []) == 0.0)
    # and they add to the routed output: y(shared) - y(no shared) = FFN(x)
    a = mod.layer_forward(x, Wr, Wg, Wu, Wd, k=2, shared=[sh])["y"]
    b = mod.layer_forward(x, Wr, Wg, Wu, Wd, k=2)["y"]
    assert np.allclose(a - b, ffn, rtol=1e-12, atol=1e-13)


def test_shared_pins():
    check_shared()


# --------------------------------------------------------------------------------- bias update

def check_bias(mod=O):
    rng = np.random.default_rng(9)
    E, k, T = 10, 3, 40                  # mean load 12
    b = (rng.random(E) * 0.1 - 0.05).astype(np.float32)
    n = np.array([12, 0, 30, 11, 13, 12, 5, 20, 12, 5])
    nb = mod.bias_update(b, n, k, T, 1e-3)
    assert nb.dtype == np.float32
    for e in range(E):
        step = np.float32(1e-3) * (1 if n[e] < 12 else (-1 if n[e] > 12 else 0))
        assert nb[e] == np.float32(b[e] + step)
    assert np.all(nb[n > 12] < b[n > 12]) and np.all(nb[n < 12] > b[n < 12])
    assert np.all(nb[n == 12] == b[n == 12])


def test_bias_pins():
    check_bias()


def test_bias_changes_selection_not_gates():
    l = _rand((30, 6), 12)
    g, _ = O.softmax_lse(l)
    b = np.array([0.0, 0.0, 10.0, 0.0, 0.0, 10.0])   # forces experts 2 and 5
    S = O.top_k(O.selection_scores(g, b), 2)
    assert all(set(r) == {2, 5} for r in S.tolist())
    w = O.gate_weights(g, S, True)
    for t in range(30):
        for j in range(2):
            assert math.isclose(w[t, j], g[t, S[t, j]] / (g[t, 2] + g[t, 5]), rel_tol=1e-14)


# ------------------------------------------------------------------------- workloads vs pages

def test_workload_shapes_match_pages():
    c = workloads.CONFIGS
    gm = GOLDEN["mixtral_shape"]
    assert (c["mixtral_8x7b"].E, c["mixtral_8x7b"].k, c["mixtral_8x7b"].M) == (gm["E"], gm["k"], gm["M"])
    gd = GOLDEN["deepseekmoe_16b_routing"]
    assert (c["deepseekmoe_16b"].E, c["deepseekmoe_16b"].k) == (gd["E"], gd["k"])
    gv = GOLDEN["deepseek_v2_routing"]
    assert (c["deepseek_v2"].E, c["deepseek_v2"].k) == (gv["E"], gv["k"])
    g3 = GOLDEN["sigmoid_v3_routing"]
    assert (c["sigmoid_v3"].E, c["sigmoid_v3"].scoring) == (g3["E"], g3["scoring"])
    assert all(cfg.lam == GOLDEN["aux_coefficient"]["lambda"] for cfg in c.values())


def test_workload_generator_is_seeded_and_per_expert():
    cfg = workloads.CONFIGS["tiny_fp32"]
    a = workloads.make_inputs(cfg)
    b = workloads.make_inputs(cfg)
    assert torch.equal(a.x, b.x) and torch.equal(a.W_gate, b.W_gate)
    assert torch.equal(workloads.make_expert(cfg, 3)[0], a.W_gate[3])
    cfg16 = workloads.CONFIGS["mixtral_8x7b"].with_(T=64, d=128, M=256)
    x = workloads.make_x(cfg16)
    assert x.dtype == torch.bfloat16 and x.shape == (64, 128)
    assert abs(float(x.float().std()) - 1.0) < 0.05


# ------------------------------------------------------------------ mutations must be caught

class _Mutant:
    """A copy of the oracle's namespace with one function replaced."""

    def __init__(self, **repl):
        self.__dict__.update({k: getattr(O, k) for k in dir(O) if not k.startswith("__")})
        self.__dict__.update(repl)
        # layer_forward looks its helpers up in the module, so rebind it to this namespace
        import types
        for name in ("layer_forward", "route", "layer_backward", "balance_loss_backward",
                     "layer_forward_expert_choice", "diagnostics", "layer_backward_expert_choice",
                     "layer_backward_sampled"):
            fn = getattr(O, name)
            self.__dict__[name] = types.FunctionType(fn.__code__, self.__dict__, name, fn.__defaults__)


def _no_renorm(g, S, renorm=True):
    return np.take_along_axis(O._f64(g), S, axis=1)


def _ties_high(s, k):
    s = O._f64(s)
    E = s.shape[1]
    rev = np.argsort(-s[:, ::-1], axis=1, kind="stable")[:, :k]
    return (E - 1) - rev


def _f_over_T(n, g, lse, k, lam):
    st = O.balance_stats(n, g, lse, 1, lam)
    return st


def _bias_wrong_sign(b, n, k, T, gamma):
    b32 = np.asarray(b, dtype=np.float32)
    return (b32 - np.float32(gamma) * np.sign((k * T) / b32.shape[0] - O._f64(n)).astype(np.float32)).astype(np.float32)


def _swiglu_transposed_down(X, Wg, Wu, Wd):
    X = O._f64(X)
    h = O.silu(X @ O._f64(Wg).T) * (X @ O._f64(Wu).T)
    return h @ O._f64(Wd)


def _dispatch_last_kept(S, E, C):
    # keep the LAST C tokens of each expert instead of the first C
    rev = O.dispatch(S[::-1], E, C)
    T, k = S.shape
    row = np.full((T, k), -1, dtype=np.int64)
    row[::-1] = np.where(rev["row"] >= 0, rev["row"], -1)
    out = dict(rev)
    out["row"] = row
    return out


def _lse_no_max(l):
    l = O._f64(l)
    lse = np.log(np.exp(l).sum(axis=1))
    return np.exp(l - lse[:, None]), lse


def _gate_from_biased(g, S, renorm=True):
    return O.gate_weights(g + 0.01, S, renorm)


def _gini_half(n):
    x = O._f64(n)
    return float(np.abs(x[:, None] - x[None, :]).sum() / (4.0 * x.shape[0] * x.sum()))


def _entropy_log2(probs):
    p = O._f64(probs)
    with np.errstate(divide="ignore", invalid="ignore"):
        return float(-np.where(p > 0, p * np.log2(p), 0.0).sum(axis=1).mean())


def _ec_ties_high(l, r):
    l = O._f64(l)
    T = l.shape[0]
    order = np.argsort(-l[::-1], axis=0, kind="stable")
    return np.sort(((T - 1) - order[:r, :]).T, axis=1).astype(np.int64)


def _ec_smallest(l, r):
    return O.expert_choice(-O._f64(l), r)


def _grad_no_centering(l, f, lam, z_coef, scoring="softmax"):
    l = O._f64(l)
    T, E = l.shape
    g, lse = O.softmax_lse(l)
    return g * (lam * E * O._f64(f) / T)[None, :] + z_coef * (2.0 / T) * lse[:, None] * g


def _silu_grad_wrong(z):
    z = O._f64(z)
    return 1.0 / (1.0 + np.exp(-z))


def _sigmoid_wrong_sign(l):
    l = O._f64(l)
    return 1.0 / (1.0 + np.exp(l))


def _sigmoid_unnormalised_P(g, scoring="softmax"):
    return O._f64(g)


def _shared_halved(x, shared):
    return 0.5 * O.shared_experts(x, shared)


def _combine_no_gate(T, d, row, w, out_perm, shared_out=None):
    return O.combine(T, d, row, np.ones_like(O._f64(w)), out_perm, shared_out)


def _combine_slots_reversed(T, d, row, w, out_perm, shared_out=None):
    # rows of the slots taken in reverse order while the gates keep theirs
    return O.combine(T, d, np.asarray(row)[:, ::-1], w, out_perm, shared_out)


def _combine_keeps_dropped(T, d, row, w, out_perm, shared_out=None):
    # a dropped slot (-1) read as the last row instead of adding nothing
    y = np.zeros((T, d)) if shared_out is None else O._f64(shared_out).copy()
    for t in range(T):
        for j in range(np.asarray(row).shape[1]):
            y[t] += w[t, j] * out_perm[int(row[t, j])]
    return y


@pytest.mark.parametrize("mutant,checks", [
    (dict(gate_weights=_no_renorm), [check_gates]),
    (dict(top_k=_ties_high), [check_topk]),
    (dict(balance_stats=_f_over_T), [check_stats]),
    (dict(bias_update=_bias_wrong_sign), [check_bias]),
    (dict(swiglu_expert=_swiglu_transposed_down), [check_experts]),
    (dict(dispatch=_dispatch_last_kept), [lambda m: check_dispatch(m, exhaustive=False)]),
    (dict(softmax_lse=_lse_no_max), [check_softmax]),
    (dict(gate_weights=_gate_from_biased), [check_gates]),
    (dict(sigmoid_scores=_sigmoid_wrong_sign), [check_sigmoid]),
    (dict(score_distribution=_sigmoid_unnormalised_P), [check_sigmoid_stats]),
    (dict(load_gini=_gini_half), [check_diagnostics]),
    (dict(routing_entropy=_entropy_log2), [check_diagnostics]),
    (dict(expert_choice=_ec_ties_high), [check_expert_choice]),
    (dict(expert_choice=_ec_smallest), [check_expert_choice]),
    (dict(balance_loss_grad_logits=_grad_no_centering), [check_loss_backward]),
    (dict(silu_grad=_silu_grad_wrong), [check_layer_backward]),
    (dict(silu_grad=_silu_grad_wrong), [check_layer_backward_ec]),
    (dict(expert_choice_capacity=lambda c, k, T, E: O.expert_choice_capacity(c, k, T, E) + 1),
     [check_layer_backward_ec]),
    (dict(shared_experts=_shared_halved), [check_shared]),
    (dict(combine=_combine_no_gate), [check_combine]),
    (dict(combine=_combine_slots_reversed), [check_combine]),
    (dict(combine=_combine_keeps_dropped), [check_combine]),
])
def test_planted_mistakes_are_caught(mutant, checks):
    m = _Mutant(**mutant)
    for chk in checks:
        with pytest.raises((AssertionError, ValueError, IndexError, KeyError, FloatingPointError)):
            with np.errstate(all="ignore"):
                chk(m)

"""GPU parity: every C-ABI entry point against the CPU oracle on the same seeded inputs.

Indices, loads, offsets, the permutation and the dropped set must match bit-exactly (tokens whose
top-k margin is within 1e-3 may pick another valid set, and the stages after routing are then
checked on the GPU's own selection); y within 2e-2 (bf16) / 1e-4 (fp32) max relative error;
statistics within 1e-5 relative. Sizes span several tiles and ragged tails."""
import math
import sys

import numpy as np
import pytest
import torch

import workloads
from oracle import moe_oracle as O
from parity_util import TOL_STATS, TOL_Y, check_selection, f64, max_rel_err, rel

pytestmark = pytest.mark.gpu

moe = None


@pytest.fixture(scope="module", autouse=True)
def _lib(gpu):
    global moe
    import mixture_experts_layer_loss_amd as m
    m.lib()  # raises if the HIP library is missing: there is no fallback
    moe = m


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def cfg_of(base, **kw):
    return workloads.CONFIGS[base].with_(**kw)


def to_dev(inp, dev):
    return workloads.MoEInputs(inp.cfg, inp.x.to(dev), inp.W_r.to(dev), inp.W_gate.to(dev),
                               inp.W_up.to(dev), inp.W_down.to(dev),
                               None if inp.b is None else inp.b.to(dev),
                               [tuple(t.to(dev) for t in s) for s in inp.shared])


# ------------------------------------------------------------------------------------- route

ROUTE_CASES = [
    ("tiny_fp32", {}),
    ("mixtral_8x7b", dict(T=300, d=512)),
    ("deepseekmoe_16b", dict(T=200, d=256)),
    ("deepseek_v2", dict(T=150, d=320)),
    ("mixtral_8x7b", dict(T=70, d=128, E=256, k=16)),
    ("mixtral_8x7b", dict(T=65, d=64, E=1, k=1)),
    ("mixtral_8x7b", dict(T=100, d=128, E=8, k=8)),
    ("mixtral_8x7b", dict(T=129, d=200, E=20, k=3)),
    ("skewed_capacity", dict(T=400, d=256)),
    # sigmoid scoring (with the bias of deepseek_v2 and sigmoid_v3; without it for mixtral)
    ("tiny_fp32", dict(scoring="sigmoid")),
    ("mixtral_8x7b", dict(T=300, d=512, scoring="sigmoid")),
    ("deepseek_v2", dict(T=150, d=320, scoring="sigmoid")),
    ("sigmoid_v3", dict(T=140, d=256)),
    ("mixtral_8x7b", dict(T=70, d=128, E=256, k=16, scoring="sigmoid", renorm=False)),
]


@pytest.mark.parametrize("base,kw", ROUTE_CASES)
def test_route(gpu, base, kw):
    cfg = cfg_of(base, **kw)
    say(f"[route] {cfg}")
    x = workloads.make_x(cfg)
    Wr = workloads.make_router(cfg)
    b = workloads.make_bias(cfg)
    r = moe.moe_route(x.to(gpu), Wr.to(gpu), cfg.k, None if b is None else b.to(gpu), cfg.renorm,
                      scoring=cfg.scoring)
    torch.cuda.synchronize()
    orc = O.route(O._f64(x), O._f64(Wr), cfg.k, None if b is None else O._f64(b), cfg.renorm,
                  cfg.scoring)
    idx = r["topk_idx"].cpu().numpy().astype(np.int64)
    n_ex, n_diff = check_selection(idx, orc, cfg.k)
    say(f"    exempt={n_ex} differ={n_diff}")
    # gates on the GPU's own selection
    w_ref = O.gate_weights(orc["g"], idx, cfg.renorm)
    assert max_rel_err(r["topk_w"], w_ref) < 1e-5
    # loads are the histogram of the GPU selection, bit-exact
    assert np.array_equal(r["n"].cpu().numpy(), O.expert_loads(idx, cfg.E))
    assert rel(r["gsum"], orc["probs"].sum(0)) < TOL_STATS
    assert rel(r["lse2sum"], [np.sum(orc["lse"] ** 2)]) < TOL_STATS
    assert rel(r["hsum"], [cfg.T * O.routing_entropy(orc["probs"])]) < TOL_STATS


# ---------------------------------------------------------------------------------- dispatch

@pytest.mark.parametrize("T,d,E,k,c,dtype", [
    (300, 128, 8, 2, None, torch.bfloat16),
    (1000, 64, 64, 8, None, torch.bfloat16),
    (777, 40, 16, 2, 1.0, torch.float32),
    (2000, 128, 64, 2, 1.25, torch.bfloat16),
    (130, 32, 256, 16, 0.5, torch.bfloat16),
    (64, 16, 1, 1, 0.25, torch.bfloat16),
])
def test_dispatch(gpu, T, d, E, k, c, dtype):
    say(f"[dispatch] T={T} d={d} E={E} k={k} c={c} {dtype}")
    g = torch.Generator().manual_seed(T + E)
    # skewed random selections: expert e chosen with weight ~ 1/(e+1)
    p = 1.0 / torch.arange(1, E + 1, dtype=torch.float64)
    S = torch.stack([torch.multinomial(p, k, replacement=False, generator=g) for _ in range(T)])
    S = S.to(torch.int32)
    x = torch.randn(T, d, generator=g).to(dtype)
    r = moe.moe_dispatch(x.to(gpu), S.to(gpu), E, c)
    torch.cuda.synchronize()
    C = O.capacity(c, k, T, E)
    ref = O.dispatch(S.numpy().astype(np.int64), E, C)
    assert np.array_equal(r["counts"].cpu().numpy(), O.expert_loads(S.numpy(), E))
    assert np.array_equal(r["offsets"].cpu().numpy(), ref["offsets"])
    assert np.array_equal(r["overflow"].cpu().numpy(), ref["overflow"])
    assert np.array_equal(r["inv_perm"].cpu().numpy(), ref["row"])
    P = int(ref["offsets"][-1])
    assert np.array_equal(r["perm_token"][:P].cpu().numpy(), ref["perm_token"])
    xp = r["x_perm"][:P].cpu()
    assert torch.equal(xp, x[torch.from_numpy(ref["perm_token"])])
    say(f"    kept={P} dropped={int(ref['overflow'].sum())}")


# -------------------------------------------------------------------------------- expert FFN

@pytest.mark.parametrize("sizes,d,Mg,dtype", [
    ([300, 0, 1, 256, 257, 513, 0, 40], 256, 384, torch.bfloat16),
    ([100, 200], 200, 136, torch.bfloat16),          # K and N tails (200 = 3*64 + 8; 136 = 128 + 8)
    ([1000], 128, 256, torch.bfloat16),
    ([70, 0, 64, 3], 128, 96, torch.float32),
    ([0, 0, 5], 64, 64, torch.bfloat16),
    # every tile class and its boundaries: remainders of 64, 65, 127, 128, 129, 192 rows
    ([383, 129, 192, 65, 64, 128, 320, 449, 0, 640], 256, 384, torch.bfloat16),
    ([64, 65, 127, 128, 129, 1], 200, 136, torch.bfloat16),   # with K and N tails
])
def test_expert_ffn(gpu, sizes, d, Mg, dtype):
    say(f"[expert_ffn] sizes={sizes} d={d} Mg={Mg} {dtype}")
    G = len(sizes)
    g = torch.Generator().manual_seed(sum(sizes) + d)
    R = sum(sizes)
    rows = torch.randn(R + 7, d, generator=g).to(dtype)  # 7 spare rows past the last group
    Wg = (torch.randn(G, Mg, d, generator=g) / math.sqrt(d)).to(dtype)
    Wu = (torch.randn(G, Mg, d, generator=g) / math.sqrt(d)).to(dtype)
    Wd = (torch.randn(G, d, Mg, generator=g) / math.sqrt(Mg)).to(dtype)
    off = torch.tensor([0] + list(np.cumsum(sizes)), dtype=torch.int32)
    h, out = moe.moe_expert_ffn(rows.to(gpu), off.to(gpu), Wg.to(gpu), Wu.to(gpu), Wd.to(gpu))
    torch.cuda.synchronize()
    tol = TOL_Y["f32" if dtype == torch.float32 else "bf16"]
    for gi in range(G):
        a, b_ = int(off[gi]), int(off[gi + 1])
        if a == b_:
            continue
        X = O._f64(rows[a:b_])
        Gm = X @ O._f64(Wg[gi]).T
        h_ref = O.silu(Gm) * (X @ O._f64(Wu[gi]).T)
        assert max_rel_err(h[a:b_], h_ref) < tol, gi
        # down projection checked on the GPU's own h (isolates the second GEMM)
        out_ref = f64(h[a:b_]) @ O._f64(Wd[gi]).T
        assert max_rel_err(out[a:b_], out_ref) < tol, gi
        full = O.swiglu_expert(X, Wg[gi], Wu[gi], Wd[gi])
        assert max_rel_err(out[a:b_], full) < tol, gi


# ----------------------------------------------------------------------------------- combine

@pytest.mark.parametrize("T,d,k,shared,dtype", [
    (333, 256, 2, False, torch.bfloat16),
    (100, 512, 8, True, torch.bfloat16),
    (77, 64, 6, True, torch.float32),
])
def test_combine(gpu, T, d, k, shared, dtype):
    say(f"[combine] T={T} d={d} k={k} shared={shared} {dtype}")
    g = torch.Generator().manual_seed(T * k)
    R = T * k
    out_perm = torch.randn(R, d, generator=g).to(dtype)
    inv = torch.randperm(R, generator=g)[: T * k].reshape(T, k).to(torch.int32)
    inv[torch.rand(T, k, generator=g) < 0.2] = -1
    inv[5] = -1  # a token with every slot dropped
    w = torch.rand(T, k, generator=g)
    sh = torch.randn(T, d, generator=g).to(dtype) if shared else None
    y = moe.moe_combine(out_perm.to(gpu), inv.to(gpu), w.to(gpu),
                        None if sh is None else sh.to(gpu))
    torch.cuda.synchronize()
    ref = O.combine(T, d, inv.numpy(), O._f64(w), O._f64(out_perm), None if sh is None else O._f64(sh))
    assert max_rel_err(y, ref) < TOL_Y["f32" if dtype == torch.float32 else "bf16"] / 4


# ------------------------------------------------------------------------------ statistics

def test_balance_stats(gpu):
    say("[balance_stats]")
    rng = np.random.default_rng(3)
    T, E, k = 5000, 160, 6
    n = rng.multinomial(k * T, np.ones(E) / E).astype(np.int32)
    n[:3] = k * T // E  # k T / E = 187.5 here, never an integer: no zero step
    gsum = rng.random(E) * T / E
    lse2 = np.array([T * 9.3])
    hsum = np.array([T * 4.1])
    b = (rng.random(E) * 0.1 - 0.05).astype(np.float32)
    dev = gpu
    r = moe.moe_balance_stats(T, k, torch.from_numpy(n).to(dev), torch.from_numpy(gsum).to(dev),
                              torch.from_numpy(lse2).to(dev), 0.01, torch.from_numpy(b).to(dev), 1e-3,
                              hsum=torch.from_numpy(hsum).to(dev))
    torch.cuda.synchronize()
    # diagnostics from the same fp64 inputs: float32 rounding of fp64 results
    dg = r["diag"].cpu().numpy().astype(np.float64)
    ref = [hsum[0] / T, O.load_gini(n), O.load_max_over_mean(n), O.importance_cv2(gsum)]
    assert np.allclose(dg, ref, rtol=1e-6, atol=0), (dg, ref)
    g_fake = np.zeros((T, E))
    g_fake[0] = gsum  # sum over tokens = gsum
    st = O.balance_stats(n, g_fake, np.sqrt(np.full(T, lse2[0] / T)), k, 0.01)
    assert rel(r["f"], st["f"]) < TOL_STATS
    assert rel(r["P"], st["P"]) < TOL_STATS
    assert rel(r["aux"], [st["aux"]]) < TOL_STATS
    assert rel(r["z"], [st["z"]]) < TOL_STATS
    assert np.array_equal(r["b_new"].cpu().numpy(), O.bias_update(b, n, k, T, 1e-3))
    # an exactly balanced expert keeps its bias (sign(0) = 0)
    T2, E2, k2 = 64, 8, 2
    n2 = np.full(E2, k2 * T2 // E2, dtype=np.int32)
    n2[0] += 1
    n2[1] -= 1
    b2 = np.linspace(-0.04, 0.04, E2).astype(np.float32)
    r2 = moe.moe_balance_stats(T2, k2, torch.from_numpy(n2).to(dev),
                               torch.ones(E2, dtype=torch.float64, device=dev) * T2 / E2,
                               torch.tensor([1.0], dtype=torch.float64, device=dev), 0.01,
                               torch.from_numpy(b2).to(dev), 1e-3)
    torch.cuda.synchronize()
    nb = r2["b_new"].cpu().numpy()
    assert nb[0] == np.float32(b2[0] - np.float32(1e-3)) and nb[1] == np.float32(b2[1] + np.float32(1e-3))
    assert np.array_equal(nb[2:], b2[2:])


# --------------------------------------------------------------------- balance-loss backward

LOSS_BW_CASES = [
    ("tiny_fp32", {}),
    ("mixtral_8x7b", dict(T=300, d=256)),
    ("deepseek_v2", dict(T=200, d=320, scoring="sigmoid")),
    ("expert_choice", dict(T=250, d=128, E=20, k=3)),
    ("mixtral_8x7b", dict(T=70, d=64, E=256, k=16)),
    ("deepseek_v2", dict(T=3000, d=320)),   # dW_r over 11 token ranges
]


@pytest.mark.parametrize("base,kw", LOSS_BW_CASES)
def test_balance_loss_backward(gpu, base, kw):
    """Gradients of aux + z_coef z through the router against the fp64 oracle (f fixed at given
    loads). Bound: the logits carry fp32 accumulation error (~1e-6 relative) and dW_r sums T fp32
    products, so 2e-4 in the max relative error of every output (R17 measure)."""
    cfg = cfg_of(base, **kw)
    say(f"[loss backward] {cfg}")
    x = workloads.make_x(cfg)
    Wr = workloads.make_router(cfg)
    rng = np.random.default_rng(7)
    fden = cfg.k * cfg.T
    n = rng.multinomial(fden, np.ones(cfg.E) / cfg.E).astype(np.int32)
    if cfg.routing == "expert":  # loads are r each
        r = O.expert_choice_capacity(cfg.c, cfg.k, cfg.T, cfg.E)
        n = np.full(cfg.E, r, dtype=np.int32)
        fden = cfg.E * r
    lam, zc = 0.01, 0.37
    out = moe.moe_balance_loss_backward(x.to(gpu), Wr.to(gpu), torch.from_numpy(n).to(gpu), cfg.k,
                                        lam, zc, c=cfg.c, scoring=cfg.scoring, routing=cfg.routing)
    torch.cuda.synchronize()
    ref = O.balance_loss_backward(O._f64(x), O._f64(Wr), n / fden, lam, zc, cfg.scoring)
    errs = {key: max_rel_err(out[key], ref[key]) for key in ("dlogits", "dW_r", "dx")}
    say(f"    {errs}")
    for key, e in errs.items():
        assert e < 2e-4, (key, e)


# -------------------------------------------------------------------------- layer backward

LAYER_BW_CASES = [
    ("tiny_fp32", {}),
    ("mixtral_8x7b", dict(T=300, d=256, M=192)),
    ("deepseekmoe_16b", dict(T=200, d=128, M=136, c=1.0)),        # shared experts, drops, N tail
    ("deepseek_v2", dict(T=150, d=200, M=72, scoring="sigmoid")),  # bias, sigmoid, K tail
    ("mixtral_8x7b", dict(T=100, d=64, M=64, E=6, k=3, renorm=False)),
    ("mixtral_8x7b", dict(T=1024, d=512, M=768)),                 # several 256 x 256 tiles
    ("mixtral_8x7b", dict(T=120, d=128, M=96)),   # K = 2M = 192, no tail; W_up from mid k-slice
    ("mixtral_8x7b", dict(T=8, d=64, M=64, E=16, k=1)),           # experts without rows
    ("mixtral_8x7b", dict(T=70, d=64, M=64, E=1, k=1)),           # one expert: a dense FFN
    ("mixtral_8x7b", dict(T=50, d=64, M=64, E=4, k=4)),           # k = E
    ("mixtral_8x7b", dict(T=90, d=64, M=64, E=4, k=2, c=0.01)),   # C = 1: nearly all dropped
    # dx rows over K = 2M = 8320 with >= 512 rows per expert: remainder tiles in two K halves
    ("mixtral_8x7b", dict(T=1100, d=128, M=4160, E=4, k=2)),
    # shared experts' weight gradients over four row ranges (two output tiles per product; the
    # last range ragged), summed in range order
    ("deepseekmoe_16b", dict(T=1100, d=128, M=136, c=1.0)),
    ("tiny_fp32", dict(T=70, E=1, k=1)),
    ("tiny_fp32", dict(T=90, E=4, k=2, c=0.01)),
    ("tiny_fp32", dict(T=120, M=96, S=2, c=1.0)),                         # fp32 shared experts
    ("tiny_fp32", dict(T=100, S=1, scoring="sigmoid", bias=True, renorm=False)),
]


@pytest.mark.parametrize("base,kw", LAYER_BW_CASES)
def test_layer_backward(gpu, base, kw):
    """Every gradient against the fp64 oracle fed the GPU's selection (the same staged parity as
    the forward). The GPU follows the real-valued chain: pre-activations, h, P = dy W_down and the
    router's gradients are fp32 on both layer dtypes.

    fp32 layers keep every product in fp32 (accumulation over at most a few thousand terms,
    ~1e-5 relative): bound 1e-4 in the max relative error of every output.

    bf16 layers run the dx-row and weight-gradient products on bf16 MFMA. Each term of those
    sums has exactly one factor rounded to bf16 once (dG, dU, or w h; the other factor, dy, x or
    a weight, is an exact bf16 input), so every element obeys |gpu - ref| <= (u + eps + K 2^-24)
    |terms| + 2^-20 max|terms|, u = 2^-8 the bf16 unit roundoff, eps = 1e-5 for the fp32 error of
    the value before rounding, K 2^-24 for fp32 accumulation over the K terms, |terms| the sum of
    the terms' magnitudes (the oracle's `magnitude`), and the absolute floor for a rounded factor
    that cancels to almost nothing in fp32 (a pre-activation near 0 carries an fp32 error of
    ~K 2^-24 of its own terms, which is no longer small relative to the factor). Rounding errors
    of random sign make the normwise error far smaller than that worst case: ||gpu - ref|| / ||ref||
    <= u for every output. dW_r has no rounded factor: max relative error 1e-4."""
    cfg = cfg_of(base, **kw)
    say(f"[layer backward] {cfg}")
    inp = workloads.make_inputs(cfg)
    d_ = to_dev(inp, gpu)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    dy = (torch.randn(cfg.T, cfg.d, generator=torch.Generator().manual_seed(11))).to(dt)
    out = moe.moe_layer_backward(d_.x, d_.W_r, d_.W_gate, d_.W_up, d_.W_down, dy.to(gpu), cfg.k,
                                 b=d_.b, shared=d_.shared_fused(), c=cfg.c, renorm=cfg.renorm,
                                 lam=cfg.lam, z_coef=0.3, scoring=cfg.scoring)
    torch.cuda.synchronize()
    gidx = out["topk_idx"].cpu().numpy().astype(np.int64)
    orc_route = O.route(O._f64(inp.x), O._f64(inp.W_r), cfg.k,
                        None if inp.b is None else O._f64(inp.b), cfg.renorm, cfg.scoring)
    check_selection(gidx, orc_route, cfg.k)
    shared = [tuple(O._f64(t) for t in s_) for s_ in inp.shared]
    bf16 = cfg.dtype == "bf16"
    ref = O.layer_backward(O._f64(inp.x), O._f64(inp.W_r), O._f64(inp.W_gate), O._f64(inp.W_up),
                           O._f64(inp.W_down), O._f64(dy), cfg.k,
                           b=None if inp.b is None else O._f64(inp.b), shared=shared, c=cfg.c,
                           renorm=cfg.renorm, lam=cfg.lam, z_coef=0.3, scoring=cfg.scoring,
                           topk_idx=gidx, magnitudes=bf16)
    compare_backward(cfg, out, ref)


def compare_backward(cfg, out, ref):
    """The bar of test_layer_backward: fp32 layers 1e-4 max relative error; bf16 layers dW_r 1e-4,
    every other element within its rounding bound and each output normwise within u."""
    bf16 = cfg.dtype == "bf16"
    pairs = {key: (out[key], ref[key]) for key in ("dx", "dW_r", "dW_gate", "dW_up", "dW_down")}
    mags = dict(ref["magnitude"]) if bf16 else {}
    if cfg.S > 0:
        # the S shared experts stacked: gate/up rows and down columns in expert order
        for i, key in enumerate(("dWs_gate", "dWs_up", "dWs_down")):
            ax = 1 if key == "dWs_down" else 0
            pairs[key] = (out[key], np.concatenate([g[i] for g in ref["shared"]], ax))
            if bf16:
                mags[key] = np.concatenate([g[i] for g in ref["magnitude"]["shared"]], ax)
    errs = {key: max_rel_err(a, r) for key, (a, r) in pairs.items()}
    say(f"    max rel {errs}")
    if not bf16:
        for key, e in errs.items():
            assert e < 1e-4, (key, e)
        return
    assert errs["dW_r"] < 1e-4, errs["dW_r"]
    u = 2.0 ** -8
    K = max(cfg.T, 2 * cfg.S * cfg.M, 2 * cfg.M, cfg.d)
    ratio, normwise = {}, {}
    for key, (a, r) in pairs.items():
        if key == "dW_r":
            continue
        a = a.detach().cpu().double().numpy() if torch.is_tensor(a) else a
        bound = (u + 1e-5 + K * 2.0 ** -24) * mags[key] + 2.0 ** -20 * mags[key].max()
        err = np.abs(a - r)
        ratio[key] = float((err / np.maximum(bound, 1e-300)).max())
        rn = np.linalg.norm(r)
        normwise[key] = float(np.linalg.norm(err) / rn) if rn > 0 else float(np.linalg.norm(err))
        assert (err <= bound).all(), (key, ratio[key])
        assert normwise[key] <= u, (key, normwise[key])
    say(f"    max err / bound {ratio}")
    say(f"    normwise {normwise}")


LAYER_BW_EC_CASES = [
    ("expert_choice", dict(T=200, d=128, M=136, E=16)),                       # shared experts
    ("expert_choice", dict(T=150, d=64, M=64, E=8, c=0.5, S=0)),              # uncovered tokens
    ("expert_choice", dict(T=100, d=64, M=72, E=6, renorm=False, scoring="sigmoid", S=0)),
    ("tiny_fp32", dict(routing="expert")),
]


SAVED_CASES = [
    ("deepseekmoe_16b", dict(T=200, d=128, M=136, c=1.0)),        # shared experts, drops, N tail
    ("deepseek_v2", dict(T=150, d=200, M=72, scoring="sigmoid")),  # bias, sigmoid, K tail
    ("mixtral_8x7b", dict(T=1024, d=512, M=768)),                 # several 256 x 256 tiles
    ("mixtral_8x7b", dict(T=8, d=64, M=64, E=16, k=1)),           # experts without rows
    ("expert_choice", dict(T=200, d=128, M=136, E=16)),           # expert choice, shared experts
]


@pytest.mark.parametrize("base,kw", SAVED_CASES)
def test_saved_pre_activations_change_nothing(gpu, base, kw):
    """A forward that keeps the fp32 gate/up pre-activations returns the same outputs bit for bit,
    and a backward that takes them instead of recomputing returns the same gradients bit for bit
    (the same GEMM tiles write them from the same accumulators; routing and placement are
    deterministic, so the rows line up)."""
    cfg = cfg_of(base, **kw)
    say(f"[saved pre-activations] {cfg}")
    inp = workloads.make_inputs(cfg)
    d_ = to_dev(inp, gpu)
    layer = moe.MoELayer(cfg.T, cfg.d, cfg.E, cfg.k, cfg.M, cfg.S, cfg.c, cfg.renorm,
                         torch.bfloat16, gpu, cfg.scoring, cfg.routing)
    saved = layer.saved_buffer()
    saved.fill_(0xFF)  # NaN patterns wherever the forward would fail to write
    a = layer.forward(d_.x, d_.W_r, d_.W_gate, d_.W_up, d_.W_down, d_.b, d_.shared_fused(), cfg.lam,
                      cfg.gamma)
    b = layer.forward(d_.x, d_.W_r, d_.W_gate, d_.W_up, d_.W_down, d_.b, d_.shared_fused(), cfg.lam,
                      cfg.gamma, out=layer.alloc_outputs(with_bias=d_.b is not None), saved=saved)
    torch.cuda.synchronize()
    keys = ["y", "counts", "f", "P", "aux", "z", "diag"]
    if cfg.routing == "token":
        keys += ["topk_idx", "topk_w"]
    for key in keys:
        assert torch.equal(a[key], b[key]), key
    dy = torch.randn(cfg.T, cfg.d, generator=torch.Generator().manual_seed(11)).to(torch.bfloat16)
    kwargs = dict(b=d_.b, shared=d_.shared_fused(), c=cfg.c, renorm=cfg.renorm, lam=cfg.lam,
                  z_coef=0.3, scoring=cfg.scoring, routing=cfg.routing)
    g0 = moe.moe_layer_backward(d_.x, d_.W_r, d_.W_gate, d_.W_up, d_.W_down, dy.to(gpu), cfg.k,
                                **kwargs)
    g1 = moe.moe_layer_backward(d_.x, d_.W_r, d_.W_gate, d_.W_up, d_.W_down, dy.to(gpu), cfg.k,
                                saved=saved, **kwargs)
    torch.cuda.synchronize()
    for key, v in g0.items():
        if key == "topk_idx" and cfg.routing == "expert":
            continue  # not written under expert choice
        assert torch.equal(v, g1[key]), key


@pytest.mark.parametrize("base,kw", LAYER_BW_EC_CASES)
def test_layer_backward_expert_choice(gpu, base, kw):
    """The expert-choice backward against the oracle's (its own selection: each case is checked to
    have no expert whose r-th and (r+1)-th logits are within 1e-4, so fp32 and fp64 logits select
    the same tokens); the bar of test_layer_backward."""
    cfg = cfg_of(base, **kw)
    say(f"[layer backward, expert choice] {cfg}")
    inp = workloads.make_inputs(cfg)
    x64 = O._f64(inp.x)
    l = O.router_logits(x64, O._f64(inp.W_r))
    r = O.expert_choice_capacity(cfg.c, cfg.k, cfg.T, cfg.E)
    if r < cfg.T:
        col = -np.sort(-l, axis=0)
        assert (col[r - 1] - col[r]).min() > 1e-4, "ambiguous selection: choose another case"
    d_ = to_dev(inp, gpu)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    dy = (torch.randn(cfg.T, cfg.d, generator=torch.Generator().manual_seed(11))).to(dt)
    out = moe.moe_layer_backward(d_.x, d_.W_r, d_.W_gate, d_.W_up, d_.W_down, dy.to(gpu), cfg.k,
                                 shared=d_.shared_fused(), c=cfg.c, renorm=cfg.renorm,
                                 lam=cfg.lam, z_coef=0.3, scoring=cfg.scoring, routing="expert")
    torch.cuda.synchronize()
    shared = [tuple(O._f64(t) for t in s_) for s_ in inp.shared]
    ref = O.layer_backward_expert_choice(
        x64, O._f64(inp.W_r), O._f64(inp.W_gate), O._f64(inp.W_up), O._f64(inp.W_down),
        O._f64(dy), cfg.k, shared=shared, c=cfg.c, renorm=cfg.renorm, lam=cfg.lam, z_coef=0.3,
        scoring=cfg.scoring, magnitudes=cfg.dtype == "bf16")
    compare_backward(cfg, out, ref)


# ------------------------------------------------------------------------------ whole layer

def run_layer(cfg, dev, inp=None):
    inp = inp or workloads.make_inputs(cfg)
    d = to_dev(inp, dev)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    layer = moe.MoELayer(cfg.T, cfg.d, cfg.E, cfg.k, cfg.M, cfg.S, cfg.c, cfg.renorm, dt, dev,
                         cfg.scoring, cfg.routing)
    out = layer.forward(d.x, d.W_r, d.W_gate, d.W_up, d.W_down, d.b, d.shared_fused(), cfg.lam,
                        cfg.gamma, out=layer.alloc_outputs(with_bias=d.b is not None,
                                                           placement=True))
    torch.cuda.synchronize()
    return inp, out


def check_layer(cfg, inp, out, tokens=None):
    """Staged parity: selection (near ties exempt), then every later stage on the GPU's selection."""
    if cfg.routing == "expert":
        return check_layer_ec(cfg, inp, out, tokens)
    x64 = O._f64(inp.x)
    orc_route = O.route(x64, O._f64(inp.W_r), cfg.k, None if inp.b is None else O._f64(inp.b),
                        cfg.renorm, cfg.scoring)
    gidx = out["topk_idx"].cpu().numpy().astype(np.int64)
    n_ex, n_diff = check_selection(gidx, orc_route, cfg.k)

    def expert(e):  # the oracle takes each expert once
        return O._f64(inp.W_gate[e]), O._f64(inp.W_up[e]), O._f64(inp.W_down[e])

    shared = [tuple(O._f64(t) for t in s) for s in inp.shared]
    res = O.layer_forward(x64, O._f64(inp.W_r), None, None, None, cfg.k,
                          b=None if inp.b is None else O._f64(inp.b), shared=shared, c=cfg.c,
                          renorm=cfg.renorm, lam=cfg.lam, gamma=cfg.gamma, topk_idx=gidx,
                          tokens=tokens, expert_weights=expert, scoring=cfg.scoring,
                          magnitudes=True)
    assert np.array_equal(out["counts"].cpu().numpy(), res["n"])
    assert np.array_equal(out["overflow"].cpu().numpy(), res["overflow"])
    # the layer's own placement ("MoE：条件计算与路由" §3), bit-exact on every assignment: rows of
    # every (t, j), the dropped set (-1), and the token of every row, whose segment starts are the
    # prefix sums of the kept counts
    if out.get("inv_perm") is not None:
        assert np.array_equal(out["inv_perm"].cpu().numpy(), res["row"])
        P = int(res["offsets"][-1])
        assert np.array_equal(out["perm_token"][:P].cpu().numpy(), res["perm_token"])
        kept = out["counts"].cpu().numpy().astype(np.int64) - out["overflow"].cpu().numpy()
        assert np.array_equal(np.concatenate([[0], np.cumsum(kept)]), res["offsets"])
    assert max_rel_err(out["topk_w"], res["topk_w"]) < 1e-5
    y = out["y"].cpu()
    ys = y if tokens is None else y[torch.as_tensor(res["tokens"])]
    err = max_rel_err(ys, res["y"], res["magnitude"])
    err_rms = max_rel_err(ys, res["y"])  # reported: the same without the term-magnitude floor
    assert err < TOL_Y[cfg.dtype], (err, err_rms)
    assert rel(out["f"], res["f"]) < TOL_STATS
    assert rel(out["P"], res["P"]) < TOL_STATS
    assert rel(out["aux"], [res["aux"]]) < TOL_STATS
    assert rel(out["z"], [res["z"]]) < TOL_STATS
    # diagnostics: entropy within the statistics bound; Gini and max/mean come from the integer
    # loads; the importance CV^2 is Var/Mean^2 of the fp32-summed importances, whose relative
    # errors (~1e-6) perturb a small CV^2 by about 2 sqrt(CV^2) 1e-6: allow 1e-5 relative + 1e-6
    dg = out["diag"].cpu().numpy().astype(np.float64)
    rd = res["diag"]
    assert rel([dg[0]], [rd["entropy"]]) < TOL_STATS
    assert abs(dg[1] - rd["gini"]) <= 1e-6 * max(rd["gini"], 1e-3)
    assert abs(dg[2] - rd["max_over_mean"]) <= 1e-6 * rd["max_over_mean"]
    assert abs(dg[3] - rd["importance_cv2"]) <= 1e-5 * rd["importance_cv2"] + 1e-6
    if inp.b is not None:
        assert np.array_equal(out["b_new"].cpu().numpy(), res["b_new"])
    return {"y_err": err, "y_err_rms_floor": err_rms, "exempt": n_ex, "differ": n_diff,
            "dropped": int(res["overflow"].sum()), "max_load": int(res["n"].max())}


def check_layer_ec(cfg, inp, out, tokens=None, exact_ties=False):
    """Expert choice: y_t depends only on which experts took token t, so y is compared on every
    token whose membership is unambiguous: for each expert whose r-th and (r+1)-th largest oracle
    logits are closer than DELTA (the fp32 logits may order them differently), tokens with a logit
    within DELTA of that gap are set aside. With exact ties (all logits equal) both sides take the
    lowest indices and every token is compared. Loads, statistics and diagnostics on all tokens."""
    DELTA = 1e-4
    x64 = O._f64(inp.x)

    def expert(e):  # the oracle takes each expert once
        return O._f64(inp.W_gate[e]), O._f64(inp.W_up[e]), O._f64(inp.W_down[e])

    shared = [tuple(O._f64(t) for t in s) for s in inp.shared]
    res = O.layer_forward_expert_choice(x64, O._f64(inp.W_r), None, None, None, cfg.k,
                                        shared=shared, c=cfg.c, renorm=cfg.renorm, lam=cfg.lam,
                                        tokens=tokens, expert_weights=expert, scoring=cfg.scoring,
                                        magnitudes=True)
    T, E, r = cfg.T, cfg.E, res["r"]
    l = res["logits"]
    srt = -np.sort(-l, axis=0)
    hi = srt[r - 1]
    lo = srt[r] if r < T else np.full(E, -np.inf)
    near = (hi - lo) < DELTA
    amb = np.any(near[None, :] & (l >= lo[None, :] - DELTA) & (l <= hi[None, :] + DELTA), axis=1)
    if exact_ties:
        amb[:] = False
    want = res["tokens"]
    sure = ~amb[want]
    assert np.all(out["counts"].cpu().numpy() == r) and np.all(out["overflow"].cpu().numpy() == 0)
    # each expert's rows hold its r tokens in ascending order; exact for every expert whose r-th
    # and (r+1)-th logits are not near a tie (all of them with exact ties)
    if out.get("perm_token") is not None:
        pt = out["perm_token"][: E * r].cpu().numpy().reshape(E, r)
        for e in range(E):
            if exact_ties or not near[e]:
                assert np.array_equal(pt[e], res["chosen"][e]), e
            else:
                assert np.all(np.diff(pt[e]) > 0) and pt[e].min() >= 0 and pt[e].max() < T
    # tokens no expert took carry only the shared term: exactly 0 without shared experts; they
    # are checked apart so that their zeros do not deflate the RMS floor of the error measure
    taken = np.zeros(T, dtype=bool)
    for e in range(E):
        taken[res["chosen"][e]] = True
    cov = taken[want] & sure
    unc = ~taken[want]
    y = out["y"].cpu()[torch.as_tensor(want)]
    mag = res["magnitude"]
    err = max_rel_err(y[torch.as_tensor(cov)], res["y"][cov], mag[cov]) if cov.any() else 0.0
    assert err < TOL_Y[cfg.dtype], err
    if unc.any():
        if cfg.S == 0:
            assert torch.all(y[torch.as_tensor(unc)] == 0)
        else:
            assert max_rel_err(y[torch.as_tensor(unc)], res["y"][unc], mag[unc]) < TOL_Y[cfg.dtype]
    assert rel(out["f"], res["f"]) < TOL_STATS
    assert rel(out["P"], res["P"]) < TOL_STATS
    assert rel(out["aux"], [res["aux"]]) < TOL_STATS
    assert rel(out["z"], [res["z"]]) < TOL_STATS
    dg = out["diag"].cpu().numpy().astype(np.float64)
    rd = res["diag"]
    assert rel([dg[0]], [rd["entropy"]]) < TOL_STATS
    assert dg[1] == 0.0 and dg[2] == 1.0  # equal loads
    assert abs(dg[3] - rd["importance_cv2"]) <= 1e-5 * rd["importance_cv2"] + 1e-6
    return {"y_err": err, "compared": int(sure.sum()), "set_aside": int((~sure).sum()), "r": r,
            "uncovered": res["uncovered"]}


LAYER_CASES = [
    ("tiny_fp32", {}),
    ("mixtral_8x7b", dict(T=1200, d=256, M=384)),
    ("deepseekmoe_16b", dict(T=700, d=192, M=200)),
    ("deepseek_v2", dict(T=600, d=320, M=136)),
    ("skewed_capacity", dict(T=2000, d=256, M=256)),
    ("mixtral_8x7b", dict(T=333, d=200, M=136, E=5, k=2)),   # K tail (200) and N tail (136)
    ("deepseekmoe_16b", dict(T=100, d=64, M=64, renorm=False)),
    ("tiny_fp32", dict(scoring="sigmoid")),
    ("deepseek_v2", dict(T=600, d=320, M=136, scoring="sigmoid")),
    ("sigmoid_v3", dict(T=700, d=256, M=128)),
    # down products over 128 k-slices with >= 512 rows per expert: remainder tiles in two K chunks
    # (64-row class, N tail 264 = 256 + 8; skewed loads with 64- and 128-row classes, K tail 8200)
    ("mixtral_8x7b", dict(T=2100, d=264, M=8256, E=4, k=2)),
    ("skewed_capacity", dict(T=2400, d=128, M=8200, E=4, k=2, c=None)),
    # expert choice: shared experts; fp32; ragged K/N tails with uncovered tokens; sigmoid scores
    ("expert_choice", dict(T=600, d=256, M=128)),
    ("tiny_fp32", dict(routing="expert")),
    ("expert_choice", dict(T=333, d=200, M=136, E=5, k=2, S=0, c=0.5)),
    ("expert_choice", dict(T=300, d=128, M=64, E=8, S=1, scoring="sigmoid")),
    ("expert_choice", dict(T=200, d=64, M=64, E=256, k=8, S=0)),
    # expert choice over more than one 8192-token chunk of the selection walk
    ("expert_choice", dict(T=9000, d=64, M=64, E=8, k=2, S=0)),
]


@pytest.mark.parametrize("base,kw", LAYER_CASES)
def test_layer(gpu, base, kw):
    cfg = cfg_of(base, **kw)
    say(f"[layer] {cfg}")
    inp, out = run_layer(cfg, gpu)
    info = check_layer(cfg, inp, out)
    say(f"    {info}")


def test_expert_choice_exact_ties(gpu):
    # a zero router: every logit is 0, so every expert takes the first r tokens on both sides
    cfg = cfg_of("expert_choice", T=257, d=64, M=64, E=6, k=2, S=0)
    say(f"[expert choice ties] {cfg}")
    inp = workloads.make_inputs(cfg)
    inp = workloads.MoEInputs(cfg, inp.x, torch.zeros_like(inp.W_r), inp.W_gate, inp.W_up,
                              inp.W_down, inp.b, inp.shared)
    _, out = run_layer(cfg, gpu, inp)
    info = check_layer_ec(cfg, inp, out, exact_ties=True)
    assert info["uncovered"] > 0 and info["set_aside"] == 0
    say(f"    {info}")


def test_layer_is_deterministic(gpu):
    cfg = cfg_of("deepseek_v2", T=300, d=256, M=128)
    say(f"[determinism] {cfg}")
    inp, a = run_layer(cfg, gpu)
    _, b = run_layer(cfg, gpu, inp)
    for key in ("y", "topk_idx", "topk_w", "counts", "f", "P", "aux", "z", "b_new"):
        assert torch.equal(a[key], b[key]), key



def test_stage_events_leave_outputs_unchanged(gpu):
    # the profiling hook (used by bench.py for per-stage times) records events and nothing else
    cfg = cfg_of("deepseekmoe_16b", T=512, d=256, M=128)
    say(f"[stage events] {cfg}")
    inp, a = run_layer(cfg, gpu)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(moe.STAGE_COUNT)]
    moe.moe_set_stage_events(evs)
    try:
        _, b = run_layer(cfg, gpu, inp)
    finally:
        moe.moe_set_stage_events(None)
    for key in ("y", "topk_idx", "topk_w", "counts", "f", "P", "aux", "z"):
        assert torch.equal(a[key], b[key]), key
    stage_ms = [evs[i].elapsed_time(evs[i + 1]) for i in range(moe.STAGE_COUNT - 1)]
    assert all(t >= 0.0 for t in stage_ms), stage_ms
    total = evs[0].elapsed_time(evs[-1])
    assert abs(sum(stage_ms) - total) <= 1e-3 + 1e-6 * total, (stage_ms, total)

def test_saved_forward_bias_survives_an_in_place_update(gpu):
    """A training forward that updates the bias in place (b_new aliasing b) keeps the bias it
    selected with in its saved buffer; the backward given that buffer selects as the forward did
    and returns the gradients of the recomputing backward at the forward's bias, bit for bit."""
    cfg = cfg_of("deepseek_v2", T=300, d=128, M=72, gamma=0.05)
    say(f"[saved bias] {cfg}")
    inp = workloads.make_inputs(cfg)
    d_ = to_dev(inp, gpu)
    b0 = d_.b.clone()
    layer = moe.MoELayer(cfg.T, cfg.d, cfg.E, cfg.k, cfg.M, cfg.S, cfg.c, cfg.renorm,
                         torch.bfloat16, gpu, cfg.scoring, cfg.routing)
    saved = layer.saved_buffer()
    b = d_.b.clone()
    out = layer.alloc_outputs(with_bias=True)
    out["b_new"] = b  # in place
    layer.forward(d_.x, d_.W_r, d_.W_gate, d_.W_up, d_.W_down, b, d_.shared_fused(), cfg.lam,
                  cfg.gamma, out=out, saved=saved)
    torch.cuda.synchronize()
    assert not torch.equal(b, b0)
    dy = torch.randn(cfg.T, cfg.d, generator=torch.Generator().manual_seed(11)).to(torch.bfloat16)
    kw = dict(shared=d_.shared_fused(), c=cfg.c, renorm=cfg.renorm, lam=cfg.lam, z_coef=0.3,
              scoring=cfg.scoring)
    args = (d_.x, d_.W_r, d_.W_gate, d_.W_up, d_.W_down, dy.to(gpu), cfg.k)
    g_saved = moe.moe_layer_backward(*args, b=b, saved=saved, **kw)
    g_ref = moe.moe_layer_backward(*args, b=b0, **kw)
    g_new = moe.moe_layer_backward(*args, b=b, **kw)
    torch.cuda.synchronize()
    for key, v in g_ref.items():
        assert torch.equal(v, g_saved[key]), key
    # the updated bias selects differently, so the kept copy is what made them equal
    assert not torch.equal(g_new["topk_idx"], g_ref["topk_idx"])
    say(f"    selections changed by the update: "
        f"{int((g_new['topk_idx'] != g_ref['topk_idx']).any(1).sum())} tokens")


def test_layer_all_dropped_gives_shared_only(gpu):
    # capacity 1: almost every slot is dropped; a token with no kept slot returns the shared term
    cfg = cfg_of("deepseekmoe_16b", T=256, d=64, M=64, c=1.0 / 128)
    say(f"[all dropped] {cfg}")
    inp, out = run_layer(cfg, gpu)
    info = check_layer(cfg, inp, out)
    assert info["dropped"] > 0
    say(f"    {info}")


# ------------------------------------------------------------------------- full-size workloads

FULL = ["tiny_fp32", "mixtral_8x7b", "deepseekmoe_16b", "deepseek_v2", "skewed_capacity",
        "sigmoid_v3", "expert_choice"]


@pytest.mark.slow
@pytest.mark.parametrize("name", FULL)
def test_full_size(gpu, name):
    """The bench launch configuration at full size, element by element on every token: the
    selection (near ties exempt), the layer's own placement (rows of every assignment, the dropped
    set and the token of every row, bit-exact), y, the statistics and the bias step."""
    cfg = workloads.CONFIGS[name]
    say(f"[full] {cfg}")
    inp, out = run_layer(cfg, gpu)
    info = check_layer(cfg, inp, out)
    say(f"    {info}")


FULL_BW = ["mixtral_8x7b", "deepseekmoe_16b", "deepseek_v2", "skewed_capacity", "sigmoid_v3"]


@pytest.mark.slow
@pytest.mark.parametrize("name", FULL_BW)
def test_full_size_backward_sampled(gpu, name):
    """The layer backward at full size, in the launch configuration bench.py times: dx on 8
    sampled tokens; row m of dW_gate[e] and dW_up[e] and column m of dW_down[e] for the most and
    the least loaded expert and two others (each entry is a sum over that expert's rows, computed
    on its own by the oracle); three columns of the stacked shared gradients. Each entry within
    its rounding bound and each sampled set normwise within u, as in test_layer_backward (dW_r,
    a sum over every token, is covered by the small cases and the balance-loss backward)."""
    cfg = workloads.CONFIGS[name]
    say(f"[full backward] {cfg}")
    inp = workloads.make_inputs(cfg)
    d_ = to_dev(inp, gpu)
    dy = torch.randn(cfg.T, cfg.d, generator=torch.Generator().manual_seed(11)).to(torch.bfloat16)
    out = moe.moe_layer_backward(d_.x, d_.W_r, d_.W_gate, d_.W_up, d_.W_down, dy.to(gpu), cfg.k,
                                 b=d_.b, shared=d_.shared_fused(), c=cfg.c, renorm=cfg.renorm,
                                 lam=cfg.lam, z_coef=1.0, scoring=cfg.scoring)
    torch.cuda.synchronize()
    gidx = out["topk_idx"].cpu().numpy().astype(np.int64)
    x64 = O._f64(inp.x)
    b64 = None if inp.b is None else O._f64(inp.b)
    check_selection(gidx, O.route(x64, O._f64(inp.W_r), cfg.k, b64, cfg.renorm, cfg.scoring),
                    cfg.k)
    rng = np.random.default_rng(3)
    tokens = np.sort(rng.choice(cfg.T, size=8, replace=False))
    loads = np.bincount(gidx.ravel(), minlength=cfg.E)
    used = np.nonzero(loads)[0]
    experts = [int(np.argmax(loads)), int(used[np.argmin(loads[used])])]
    experts += [int(e) for e in rng.choice(used, size=2, replace=False)]
    cols = [(e, int(m)) for e, m in zip(experts, [cfg.M - 1, 0, *rng.integers(0, cfg.M, 2)])]
    SM = cfg.S * cfg.M
    scols = [0, SM - 1, int(rng.integers(0, SM))] if cfg.S > 0 else []
    shared = [tuple(O._f64(t) for t in s_) for s_ in inp.shared]
    ref = O.layer_backward_sampled(
        x64, inp.W_r, None, None, None, dy, cfg.k, b=b64, shared=shared, c=cfg.c,
        renorm=cfg.renorm, lam=cfg.lam, z_coef=1.0, scoring=cfg.scoring, topk_idx=gidx,
        tokens=tokens, expert_cols=cols, shared_cols=scols,
        expert_weights=lambda e: (inp.W_gate[e], inp.W_up[e], inp.W_down[e]))
    got = {"dx": out["dx"][torch.as_tensor(tokens, device=gpu)].cpu().double().numpy()}
    got["dW_gate"] = [out["dW_gate"][e, m].cpu().double().numpy() for e, m in cols]
    got["dW_up"] = [out["dW_up"][e, m].cpu().double().numpy() for e, m in cols]
    got["dW_down"] = [out["dW_down"][e, :, m].cpu().double().numpy() for e, m in cols]
    if scols:
        got["dWs_gate"] = [out["dWs_gate"][m].cpu().double().numpy() for m in scols]
        got["dWs_up"] = [out["dWs_up"][m].cpu().double().numpy() for m in scols]
        got["dWs_down"] = [out["dWs_down"][:, m].cpu().double().numpy() for m in scols]
    u = 2.0 ** -8
    K = max(cfg.T, 2 * SM, 2 * cfg.M, cfg.d)
    ratio, normwise = {}, {}
    for key, val in got.items():
        a = np.asarray(val, dtype=np.float64)
        r = np.asarray(ref[key], dtype=np.float64)
        mag = np.asarray(ref["magnitude"][key], dtype=np.float64)
        err = np.abs(a - r)
        bound = (u + 1e-5 + K * 2.0 ** -24) * mag + 2.0 ** -20 * mag.max()
        ratio[key] = float((err / np.maximum(bound, 1e-300)).max())
        normwise[key] = float(np.linalg.norm(err) / np.linalg.norm(r))
        assert (err <= bound).all(), (key, ratio[key])
        assert normwise[key] <= u, (key, normwise[key])
    say(f"    experts {cols} shared {scols}")
    say(f"    max err / bound {ratio}")
    say(f"    normwise {normwise}")

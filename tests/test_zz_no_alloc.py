"""The no-allocation layer forward (moe_layer_forward_noalloc) against moe_layer_forward.

Both run the same kernels; the only difference is where the workspace lives (the library's static
scratch instead of a caller buffer), so every output must be bit-identical. Two calls in a row on
one device, the second with a smaller input, check that nothing left in the scratch by a call
reaches the next."""
import sys

import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

KEYS = ("y", "topk_idx", "topk_w", "counts", "overflow", "f", "P", "aux", "z", "diag", "inv_perm",
        "perm_token", "b_new")


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _pair(moe, cfg, dev):
    inp = workloads.make_inputs(cfg)
    x, Wr, Wg, Wu, Wd = (t.to(dev) for t in (inp.x, inp.W_r, inp.W_gate, inp.W_up, inp.W_down))
    b = None if inp.b is None else inp.b.to(dev)
    sh = inp.shared_fused()
    sh = None if sh is None else tuple(t.to(dev) for t in sh)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    ref_layer = moe.MoELayer(cfg.T, cfg.d, cfg.E, cfg.k, cfg.M, cfg.S, cfg.c, cfg.renorm, dt, dev,
                             cfg.scoring, cfg.routing)
    na_layer = moe.MoELayer(cfg.T, cfg.d, cfg.E, cfg.k, cfg.M, cfg.S, cfg.c, cfg.renorm, dt, dev,
                            cfg.scoring, cfg.routing, with_workspace=False)
    assert moe.workspace_size(na_layer.shape, moe.CALL_LAYER) <= moe.SCRATCH_BYTES
    ref = ref_layer.alloc_outputs(b is not None, placement=True)
    out = na_layer.alloc_outputs(b is not None, placement=True)
    if b is not None:
        ref["b_new"].fill_(0.0)
        out["b_new"].fill_(0.0)
    ref = ref_layer.forward(x, Wr, Wg, Wu, Wd, b, sh, cfg.lam, cfg.gamma, out=ref)
    got = na_layer.forward(x, Wr, Wg, Wu, Wd, b, sh, cfg.lam, cfg.gamma, out=out, noalloc=True)
    torch.cuda.synchronize()
    for key in KEYS:
        if cfg.routing == "expert" and key in ("topk_idx", "topk_w"):
            continue  # not written under expert choice
        if ref.get(key) is None:
            assert got.get(key) is None, key
            continue
        assert torch.equal(ref[key], got[key]), key


@pytest.mark.parametrize("first,second", [
    # Mixtral-shaped (T=600: 44 MB of scratch), then a smaller layer
    (("mixtral_8x7b", dict(T=600)), ("mixtral_8x7b", dict(T=129, d=512, M=768))),
    # shared experts, a bias, sigmoid scores and capacity drops, then a smaller one
    (("deepseek_v2", dict(T=256, d=1024, M=512, c=1.0)), ("deepseek_v2", dict(T=40, d=256, M=64))),
    # expert choice, then fp32
    (("expert_choice", dict(T=300, d=512, M=256)), ("tiny_fp32", dict(T=100))),
])
def test_noalloc_forward_matches_allocating_forward(gpu, first, second):
    import mixture_experts_layer_loss_amd as moe
    moe.lib()
    for base, kw in (first, second):
        cfg = workloads.CONFIGS[base].with_(**kw)
        _say(f"[noalloc] {cfg}")
        _pair(moe, cfg, gpu)

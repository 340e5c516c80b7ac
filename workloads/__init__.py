"""Seeded synthetic inputs for the sparse MoE FFN layer (shared by the oracle and the HIP path).

This module holds only input generation: shapes, seeds and value distributions. It contains
none of the layer's arithmetic (no routing, softmax, top-k, dispatch, expert FFN or statistics),
so that the CPU oracle and the GPU path can both be fed from it without sharing any method code.

Workloads (shapes taken from the models the source pages name):

* ``tiny_fp32``        T=256,   d=128,  E=8,   k=2, M=256,   fp32 (correctness case)
* ``mixtral_8x7b``     T=4096,  d=4096, E=8,   k=2, M=14336, bf16 -- Mixtral 8x7B layer shape
                       ("MoE：条件计算与路由", §细粒度专家分割, eqs. (1)-(3): E=8, k=2, M=14336)
* ``deepseekmoe_16b``  T=8192,  d=2048, E=64,  k=8, M=1408,  S=2 shared, bf16
                       ("MOE大模型对比篇", §3.2 fine-grained segmentation, 64 experts choose 8;
                       §3.3 shared-expert isolation)
* ``deepseek_v2``      T=16384, d=5120, E=160, k=6, M=1536,  S=2 shared, bf16, per-expert
                       loss-free-balancing bias b_e ~ U(-0.05, 0.05), update rate gamma=1e-3
                       ("MoE" (t4mako), §DeepSeek V2 的 MoE 创新: 160 small experts choose 6 plus
                       shared experts; "MoE：条件计算与路由", §无辅助损失负载均衡（ALF-LB）)
* ``skewed_capacity``  T=32768, d=4096, E=64,  k=2, M=2048,  bf16, capacity factor c=1.25
                       ("MoE：条件计算与路由", §3 Capacity factor 和 token dropping), with router
                       logits skewed by per-expert Zipf(1.2) offsets so the hottest expert receives
                       about 8x the mean load.

Distributions: x ~ N(0,1); W_r ~ N(0,1/d); W_gate, W_up ~ N(0,1/d); W_down ~ N(0,1/M) (shared
experts likewise). Every tensor, and every expert's slice of an expert tensor, has its own
torch CPU generator seeded from (seed, tensor id, expert), so any one expert can be regenerated
alone. bf16 workloads draw fp32 values and round them once to bf16 (round-to-nearest-even).

Zipf skew (``skewed_capacity``): expert e gets rank r_e = pi(e)+1 from a seeded permutation pi, and
the logit offset o_e = alpha * ln(r_e^-s / H) with H = sum_r r^-s. The offset is folded into the
router by fixing input feature 0 to 1.0 for every token and adding o_e to W_r[e, 0] before the
bf16 rounding, so the logits carry the per-expert offsets without any extra argument. alpha is a
stored constant (``zipf_alpha.json``) written by ``oracle/calibrate_zipf.py``.
"""
from __future__ import annotations

import json
import math
import os
from dataclasses import dataclass, field, replace
from typing import Dict, Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int            # tokens in the routing batch (B on the pages)
    d: int            # hidden size
    E: int            # routed experts
    k: int            # experts chosen per token
    M: int            # expert intermediate width
    S: int = 0        # shared experts (each of width M), applied to every token
    c: Optional[float] = None   # capacity factor; None = dropless
    dtype: str = "bf16"         # "bf16" or "f32": x, weights, intermediates and y
    bias: bool = False          # draw a loss-free-balancing bias b_e ~ U(-0.05, 0.05)
    gamma: float = 1e-3         # bias update rate
    lam: float = 0.01           # aux-loss coefficient lambda
    renorm: bool = True         # renormalise the top-k gates
    zipf_s: Optional[float] = None  # Zipf exponent of the router-logit skew (None = none)
    seed: int = 0
    scoring: str = "softmax"    # router scores: "softmax" or per-expert "sigmoid"
    routing: str = "token"      # "token" choice (top-k experts) or "expert" choice (top-r tokens)

    def with_(self, **kw) -> "MoEConfig":
        return replace(self, **kw)


CONFIGS: Dict[str, MoEConfig] = {
    "tiny_fp32": MoEConfig("tiny_fp32", T=256, d=128, E=8, k=2, M=256, dtype="f32"),
    "mixtral_8x7b": MoEConfig("mixtral_8x7b", T=4096, d=4096, E=8, k=2, M=14336),
    "deepseekmoe_16b": MoEConfig("deepseekmoe_16b", T=8192, d=2048, E=64, k=8, M=1408, S=2),
    "deepseek_v2": MoEConfig("deepseek_v2", T=16384, d=5120, E=160, k=6, M=1536, S=2, bias=True),
    "skewed_capacity": MoEConfig("skewed_capacity", T=32768, d=4096, E=64, k=2, M=2048, c=1.25,
                                 zipf_s=1.2),
    # the DeepSeek-V3 gate: 256 routed experts scored by a sigmoid, loss-free-balancing bias, one
    # shared expert; hidden and expert widths as the DeepSeek-V2 layer above, 8 chosen per token
    "sigmoid_v3": MoEConfig("sigmoid_v3", T=16384, d=5120, E=256, k=8, M=1536, S=1, bias=True,
                            scoring="sigmoid"),
    # expert-choice routing on the DeepSeekMoE layer: 64 experts each take r = 2 T / 64 tokens
    # (the same number of assignments as top-2 token choice), two shared experts
    "expert_choice": MoEConfig("expert_choice", T=8192, d=2048, E=64, k=2, M=1408, S=2,
                               routing="expert"),
}

# the configuration the headline metric is quoted on
HEADLINE = "mixtral_8x7b"

_TID = {"x": 1, "W_r": 2, "W_gate": 3, "W_up": 4, "W_down": 5,
        "Ws_gate": 6, "Ws_up": 7, "Ws_down": 8, "b": 9, "zipf_perm": 10}


def _gen(seed: int, tensor: str, part: int = 0) -> torch.Generator:
    s = (int(seed) * 1_000_003 + _TID[tensor] * 65_537 + int(part) * 977) & ((1 << 62) - 1)
    return torch.Generator().manual_seed(s)


def _normal(shape, std: float, g: torch.Generator) -> torch.Tensor:
    return torch.randn(*shape, generator=g, dtype=torch.float32).mul_(std)


def _store(t: torch.Tensor, cfg: MoEConfig) -> torch.Tensor:
    return t.to(torch.bfloat16) if cfg.dtype == "bf16" else t.contiguous()


def zipf_alpha(cfg: MoEConfig) -> float:
    """The stored Zipf-offset scale for ``cfg`` (0.0 when the config has no skew)."""
    if cfg.zipf_s is None:
        return 0.0
    path = os.path.join(_HERE, "zipf_alpha.json")
    with open(path) as fh:
        table = json.load(fh)
    key = f"{cfg.name}:s={cfg.zipf_s}"
    if key not in table:
        raise KeyError(f"no calibrated Zipf alpha for {key}; run oracle/calibrate_zipf.py")
    return float(table[key]["alpha"])


def zipf_offsets(cfg: MoEConfig, alpha: Optional[float] = None) -> torch.Tensor:
    """Per-expert logit offsets o_e = alpha * ln(r_e^-s / H), fp32 [E]."""
    if cfg.zipf_s is None:
        return torch.zeros(cfg.E)
    a = zipf_alpha(cfg) if alpha is None else float(alpha)
    perm = torch.randperm(cfg.E, generator=_gen(cfg.seed, "zipf_perm"))
    ranks = perm.to(torch.float64) + 1.0
    H = sum(r ** (-cfg.zipf_s) for r in range(1, cfg.E + 1))
    o = a * torch.log(ranks.pow(-cfg.zipf_s) / H)
    return o.to(torch.float32)


def make_x(cfg: MoEConfig) -> torch.Tensor:
    x = _normal((cfg.T, cfg.d), 1.0, _gen(cfg.seed, "x"))
    if cfg.zipf_s is not None:
        x[:, 0] = 1.0
    return _store(x, cfg)


def make_router(cfg: MoEConfig, alpha: Optional[float] = None) -> torch.Tensor:
    w = _normal((cfg.E, cfg.d), 1.0 / math.sqrt(cfg.d), _gen(cfg.seed, "W_r"))
    if cfg.zipf_s is not None:
        w[:, 0] += zipf_offsets(cfg, alpha)
    return _store(w, cfg)


def make_expert(cfg: MoEConfig, e: int, shared: bool = False):
    """(W_gate [M,d], W_up [M,d], W_down [d,M]) of routed expert e, or of shared expert e."""
    pre = "Ws_" if shared else "W_"
    Wg = _normal((cfg.M, cfg.d), 1.0 / math.sqrt(cfg.d), _gen(cfg.seed, pre + "gate", e))
    Wu = _normal((cfg.M, cfg.d), 1.0 / math.sqrt(cfg.d), _gen(cfg.seed, pre + "up", e))
    Wd = _normal((cfg.d, cfg.M), 1.0 / math.sqrt(cfg.M), _gen(cfg.seed, pre + "down", e))
    return _store(Wg, cfg), _store(Wu, cfg), _store(Wd, cfg)


def make_bias(cfg: MoEConfig) -> Optional[torch.Tensor]:
    if not cfg.bias:
        return None
    g = _gen(cfg.seed, "b")
    return (torch.rand(cfg.E, generator=g, dtype=torch.float32) * 0.1 - 0.05).contiguous()


@dataclass
class MoEInputs:
    cfg: MoEConfig
    x: torch.Tensor                 # [T, d]
    W_r: torch.Tensor               # [E, d]
    W_gate: torch.Tensor            # [E, M, d]
    W_up: torch.Tensor              # [E, M, d]
    W_down: torch.Tensor            # [E, d, M]
    b: Optional[torch.Tensor]       # [E] fp32 or None
    shared: list = field(default_factory=list)  # S tuples (Wg [M,d], Wu [M,d], Wd [d,M])

    def shared_fused(self):
        """The S shared experts as one expert of width S*M (gate/up stacked along M, down along
        its input dimension), or None when S == 0."""
        if not self.shared:
            return None
        Wg = torch.cat([s[0] for s in self.shared], 0).contiguous()
        Wu = torch.cat([s[1] for s in self.shared], 0).contiguous()
        Wd = torch.cat([s[2] for s in self.shared], 1).contiguous()
        return Wg, Wu, Wd


def make_inputs(cfg: MoEConfig, alpha: Optional[float] = None, device: Optional[str] = None) -> MoEInputs:
    """All inputs of one layer forward, on the CPU (or moved to ``device`` expert by expert)."""
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    dev = torch.device(device) if device is not None else torch.device("cpu")
    Wg = torch.empty((cfg.E, cfg.M, cfg.d), dtype=dt, device=dev)
    Wu = torch.empty((cfg.E, cfg.M, cfg.d), dtype=dt, device=dev)
    Wd = torch.empty((cfg.E, cfg.d, cfg.M), dtype=dt, device=dev)
    for e in range(cfg.E):
        g, u, dn = make_expert(cfg, e)
        Wg[e].copy_(g)
        Wu[e].copy_(u)
        Wd[e].copy_(dn)
    shared = [tuple(t.to(dev) for t in make_expert(cfg, s, shared=True)) for s in range(cfg.S)]
    b = make_bias(cfg)
    return MoEInputs(cfg, make_x(cfg).to(dev), make_router(cfg, alpha).to(dev), Wg, Wu, Wd,
                     None if b is None else b.to(dev), shared)

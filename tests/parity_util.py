"""Comparison helpers for GPU-vs-oracle parity.

* ``max_rel_err(a, r, mag)`` = max_i |a_i - r_i| / max(|r_i|, rms(r), mag_i): elementwise
  relative error, floored at the reference RMS so that near-zero reference elements do not
  dominate, and, for the layer output, at the magnitude of the terms summed into it (mag_i =
  sum of |w E(x)| over the combine's terms plus the shared terms): each term is rounded to bf16
  before the sum, so an element whose terms cancel carries an error set by the terms, not by y.
* Tolerances: 2e-2 for bf16 layers (bf16 storage, fp32 accumulation), 1e-4 for fp32 layers,
  1e-5 relative for the balance statistics.
* Near ties: a token whose k-th and (k+1)-th oracle selection scores are within 1e-3 may pick a
  different (equally valid) set; for such tokens only validity is checked.
"""
import numpy as np
import torch

TOL_Y = {"bf16": 2e-2, "f32": 1e-4}
TOL_STATS = 1e-5
TIE_MARGIN = 1e-3


def f64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        t = t.detach().cpu()
        if t.dtype == torch.bfloat16:
            t = t.float()
        return t.numpy().astype(np.float64)
    return np.asarray(t, dtype=np.float64)


def max_rel_err(a, r, mag=None) -> float:
    a, r = f64(a), f64(r)
    if r.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(r * r)))
    den = np.maximum(np.abs(r), rms if rms > 0 else 1.0)
    if mag is not None:
        den = np.maximum(den, f64(mag))
    return float(np.max(np.abs(a - r) / den))


def rel(a, r) -> float:
    a, r = f64(a), f64(r)
    return float(np.max(np.abs(a - r) / np.maximum(np.abs(r), 1e-300)))


def check_selection(gpu_idx: np.ndarray, orc: dict, k: int):
    """Exact match where the oracle's top-k margin exceeds 1e-3; elsewhere the GPU's choice must
    be a valid top-k of the oracle scores (within 1e-6). Returns (n_exempt, n_differ)."""
    S_ref = orc["topk_idx"]
    s = orc["s"]
    margin = orc["margin"]
    strict = margin > TIE_MARGIN
    bad = np.where(strict & np.any(gpu_idx != S_ref, axis=1))[0]
    assert len(bad) == 0, f"{len(bad)} non-tie tokens differ, e.g. token {bad[:5]}"
    E = s.shape[1]
    for t in np.where(~strict)[0]:
        chosen = gpu_idx[t]
        assert len(set(chosen.tolist())) == k and chosen.min() >= 0 and chosen.max() < E
        rest = np.setdiff1d(np.arange(E), chosen)
        if rest.size:
            assert s[t, chosen].min() >= s[t, rest].max() - 1e-6, t
        assert np.all(np.diff(s[t, chosen]) <= 1e-6), t
    n_differ = int(np.sum(np.any(gpu_idx != S_ref, axis=1)))
    return int((~strict).sum()), n_differ

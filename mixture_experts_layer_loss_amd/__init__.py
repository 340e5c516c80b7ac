"""Python binding of the MI355X MoE layer library (``libmoe.so``, C ABI in ``include/moe.h``).

The functions below carry the C entry points' names and do argument marshalling only: they check
tensor shapes, dtypes and devices, allocate output tensors with torch (device memory is torch's
plumbing), and pass raw device pointers plus torch's current HIP stream to the library. Every step
of the layer runs in the library's HIP kernels. There is no fallback: if the library is missing or
fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "moe.h")

MOE_OK, MOE_ERR_INVALID_ARGUMENT, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP, \
    MOE_ERR_SCRATCH = range(6)
SCRATCH_BYTES = 64 << 20  # MOE_SCRATCH_BYTES: static scratch of moe_layer_forward_noalloc
MOE_F32, MOE_BF16 = 0, 1
CALL_ROUTE, CALL_DISPATCH, CALL_EXPERT_FFN, CALL_LAYER, CALL_LOSS_BACKWARD, CALL_LAYER_BACKWARD = range(6)
E_MAX, K_MAX = 256, 16


class MoEError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


class Shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("M", ctypes.c_int32), ("S", ctypes.c_int32),
                ("c", ctypes.c_float), ("renorm", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("scoring", ctypes.c_int32), ("routing", ctypes.c_int32)]


SCORING = {"softmax": 0, "sigmoid": 1}  # moe_scoring
ROUTING = {"token": 0, "expert": 1}     # moe_routing: token choice, expert choice


_P = ctypes.c_void_p
_SIG = {
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_check_shape": (ctypes.c_int, [ctypes.POINTER(Shape)]),
    "moe_capacity": (ctypes.c_int64, [ctypes.POINTER(Shape)]),
    "moe_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(Shape), ctypes.c_int]),
    "moe_saved_size": (ctypes.c_size_t, [ctypes.POINTER(Shape)]),
    "moe_routed_rows": (ctypes.c_int64, [ctypes.POINTER(Shape)]),
    "moe_route": (ctypes.c_int, [ctypes.POINTER(Shape), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                 ctypes.c_size_t, _P]),
    "moe_dispatch": (ctypes.c_int, [ctypes.POINTER(Shape), _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                    ctypes.c_size_t, _P]),
    "moe_expert_ffn": (ctypes.c_int, [ctypes.POINTER(Shape), ctypes.c_int32, ctypes.c_int32, _P,
                                      _P, ctypes.c_int64, _P, _P, _P, _P, _P, _P, ctypes.c_size_t,
                                      _P]),
    "moe_combine": (ctypes.c_int, [ctypes.POINTER(Shape), _P, _P, _P, _P, _P, _P]),
    "moe_balance_stats": (ctypes.c_int, [ctypes.POINTER(Shape), _P, _P, _P, _P, ctypes.c_float, _P,
                                         _P, _P, _P, _P, _P, _P, ctypes.c_float, _P]),
    "moe_layer_forward": (ctypes.c_int, [ctypes.POINTER(Shape), _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                         _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                         ctypes.c_float, ctypes.c_float, _P, _P, ctypes.c_size_t,
                                         _P]),
    "moe_layer_forward_noalloc": (ctypes.c_int, [ctypes.POINTER(Shape), _P, _P, _P, _P, _P, _P, _P,
                                                 _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                                 _P, _P, _P, ctypes.c_float, ctypes.c_float, _P,
                                                 _P]),
    "moe_set_stage_events": (ctypes.c_int, [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int]),
    "moe_balance_loss_backward": (ctypes.c_int, [ctypes.POINTER(Shape), _P, _P, _P, ctypes.c_float,
                                                 ctypes.c_float, _P, _P, _P, _P, ctypes.c_size_t,
                                                 _P]),
    "moe_layer_backward": (ctypes.c_int, [ctypes.POINTER(Shape), _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                          _P, ctypes.c_float, ctypes.c_float, _P, _P, _P, _P, _P,
                                          _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
}

STAGES = ["route", "dispatch", "gemm_up", "gemm_down", "shared", "combine", "stats"]
STAGE_COUNT = 8

_lib_handle = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built (there is no fallback path)."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m mixture_experts_layer_loss_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIG.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib_handle = h
    return _lib_handle


def header_functions() -> list:
    """Names of the functions declared in include/moe.h."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(moe_\w+)\s*\(", text, flags=re.M)))


def status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status != MOE_OK:
        raise MoEError(status, what)


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return MOE_BF16
    if dt == torch.float32:
        return MOE_F32
    raise TypeError(f"unsupported dtype {dt}: the library takes bfloat16 or float32")


def make_shape(T: int, d: int, E: int, k: int, M: int, S: int = 0, c: Optional[float] = None,
               renorm: bool = True, dtype: torch.dtype = torch.bfloat16,
               scoring: str = "softmax", routing: str = "token") -> Shape:
    if scoring not in SCORING:
        raise ValueError(f"scoring must be one of {sorted(SCORING)}, got {scoring!r}")
    if routing not in ROUTING:
        raise ValueError(f"routing must be one of {sorted(ROUTING)}, got {routing!r}")
    return Shape(int(T), int(d), int(E), int(k), int(M), int(S),
                 float(c) if c is not None else 0.0, 1 if renorm else 0, _dtype_code(dtype),
                 SCORING[scoring], ROUTING[routing])


def check_shape(s: Shape) -> int:
    return lib().moe_check_shape(ctypes.byref(s))


def capacity(s: Shape) -> int:
    return int(lib().moe_capacity(ctypes.byref(s)))


def workspace_size(s: Shape, call: int) -> int:
    return int(lib().moe_workspace_size(ctypes.byref(s), int(call)))


def routed_rows(s: Shape) -> int:
    """moe_routed_rows: rows of the expert-contiguous routed buffers (entries of perm_token)."""
    return int(lib().moe_routed_rows(ctypes.byref(s)))


def _shared_count(shared, M: int, d: int, dtype) -> int:
    """S from the stacked shared experts (Ws_gate [S*M, d], Ws_up [S*M, d], Ws_down [d, S*M])."""
    if shared is None:
        return 0
    if len(shared) != 3:
        raise ValueError("shared must be (Ws_gate, Ws_up, Ws_down)")
    SM = shared[0].shape[0]
    if shared[0].dim() != 2 or SM == 0 or SM % M != 0:
        raise ValueError(f"Ws_gate must be [S*M, d] with S >= 1 and M = {M}, got "
                         f"{tuple(shared[0].shape)}")
    for name, t, shp in (("Ws_gate", shared[0], (SM, d)), ("Ws_up", shared[1], (SM, d)),
                         ("Ws_down", shared[2], (d, SM))):
        _dev(t, name, dtype, shp)
    return SM // M


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def workspace(s: Shape, call: int, device) -> torch.Tensor:
    n = workspace_size(s, call)
    if n == 0:
        _check(check_shape(s), "workspace_size")
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


# --------------------------------------------------------------------------------- entry points

def moe_route(x: torch.Tensor, W_r: torch.Tensor, k: int, b: Optional[torch.Tensor] = None,
              renorm: bool = True, ws: Optional[torch.Tensor] = None,
              scoring: str = "softmax") -> dict:
    T, d = x.shape
    E = W_r.shape[0]
    s = make_shape(T, d, E, k, 8, renorm=renorm, dtype=x.dtype, scoring=scoring)
    _dev(x, "x")
    _dev(W_r, "W_r", x.dtype, (E, d))
    if b is not None:
        _dev(b, "b", torch.float32, (E,))
    dev = x.device
    out = {"topk_idx": torch.empty(T, k, dtype=torch.int32, device=dev),
           "topk_w": torch.empty(T, k, dtype=torch.float32, device=dev),
           "n": torch.empty(E, dtype=torch.int32, device=dev),
           "gsum": torch.empty(E, dtype=torch.float64, device=dev),
           "lse2sum": torch.empty(1, dtype=torch.float64, device=dev),
           "hsum": torch.empty(1, dtype=torch.float64, device=dev)}
    if ws is None:
        ws = workspace(s, CALL_ROUTE, dev)
    _check(lib().moe_route(ctypes.byref(s), _ptr(x), _ptr(W_r), _ptr(b), _ptr(out["topk_idx"]),
                           _ptr(out["topk_w"]), _ptr(out["n"]), _ptr(out["gsum"]),
                           _ptr(out["lse2sum"]), _ptr(out["hsum"]), _ptr(ws), ws.numel(),
                           _stream()), "moe_route")
    return out


def moe_dispatch(x: torch.Tensor, topk_idx: torch.Tensor, E: int, c: Optional[float] = None,
                 copy_rows: bool = True, ws: Optional[torch.Tensor] = None) -> dict:
    T, d = x.shape
    k = topk_idx.shape[1]
    s = make_shape(T, d, E, k, 8, c=c, dtype=x.dtype)
    _dev(x, "x")
    _dev(topk_idx, "topk_idx", torch.int32, (T, k))
    dev = x.device
    rows = T * k
    out = {"x_perm": torch.empty(rows, d, dtype=x.dtype, device=dev) if copy_rows else None,
           "perm_token": torch.full((rows,), -1, dtype=torch.int32, device=dev),
           "inv_perm": torch.empty(T, k, dtype=torch.int32, device=dev),
           "offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
           "counts": torch.empty(E, dtype=torch.int32, device=dev),
           "overflow": torch.empty(E, dtype=torch.int32, device=dev)}
    if ws is None:
        ws = workspace(s, CALL_DISPATCH, dev)
    _check(lib().moe_dispatch(ctypes.byref(s), _ptr(x), _ptr(topk_idx), _ptr(out["x_perm"]),
                              _ptr(out["perm_token"]), _ptr(out["inv_perm"]), _ptr(out["offsets"]),
                              _ptr(out["counts"]), _ptr(out["overflow"]), _ptr(ws), ws.numel(),
                              _stream()), "moe_dispatch")
    return out


def moe_expert_ffn(rows: torch.Tensor, offsets: torch.Tensor, W_gate: torch.Tensor,
                   W_up: torch.Tensor, W_down: torch.Tensor, ws: Optional[torch.Tensor] = None):
    """Grouped SwiGLU over row groups [offsets[g], offsets[g+1]); returns (h, out)."""
    R, d = rows.shape
    G, Mg, d2 = W_gate.shape
    if d2 != d:
        raise ValueError("W_gate must be [groups, Mg, d]")
    _dev(rows, "rows")
    _dev(offsets, "offsets", torch.int32, (G + 1,))
    _dev(W_gate, "W_gate", rows.dtype)
    _dev(W_up, "W_up", rows.dtype, (G, Mg, d))
    _dev(W_down, "W_down", rows.dtype, (G, d, Mg))
    s = make_shape(max(R, 1), d, G, 1, Mg, dtype=rows.dtype)
    h = torch.empty(R, Mg, dtype=rows.dtype, device=rows.device)
    out = torch.empty(R, d, dtype=rows.dtype, device=rows.device)
    if ws is None:
        ws = workspace(s, CALL_EXPERT_FFN, rows.device)
    _check(lib().moe_expert_ffn(ctypes.byref(s), G, Mg, _ptr(rows), _ptr(offsets), R, _ptr(W_gate),
                                _ptr(W_up), _ptr(W_down), _ptr(h), _ptr(out), _ptr(ws), ws.numel(),
                                _stream()), "moe_expert_ffn")
    return h, out


def moe_combine(out_perm: torch.Tensor, inv_perm: torch.Tensor, topk_w: torch.Tensor,
                shared_out: Optional[torch.Tensor] = None) -> torch.Tensor:
    T, k = inv_perm.shape
    d = out_perm.shape[1]
    _dev(out_perm, "out_perm")
    _dev(inv_perm, "inv_perm", torch.int32)
    _dev(topk_w, "topk_w", torch.float32, (T, k))
    if shared_out is not None:
        _dev(shared_out, "shared_out", out_perm.dtype, (T, d))
    s = make_shape(T, d, max(k, 1), k, 8, dtype=out_perm.dtype)
    y = torch.empty(T, d, dtype=out_perm.dtype, device=out_perm.device)
    _check(lib().moe_combine(ctypes.byref(s), _ptr(out_perm), _ptr(inv_perm), _ptr(topk_w),
                             _ptr(shared_out), _ptr(y), _stream()), "moe_combine")
    return y


def moe_balance_stats(T: int, k: int, n: torch.Tensor, gsum: torch.Tensor, lse2sum: torch.Tensor,
                      lam: float = 0.01, b: Optional[torch.Tensor] = None,
                      gamma: float = 1e-3, hsum: Optional[torch.Tensor] = None) -> dict:
    """Balance statistics; with ``hsum`` (from moe_route) also the routing diagnostics ``diag``:
    [mean routing entropy, load Gini, max/mean load, importance CV^2]."""
    E = n.shape[0]
    _dev(n, "n", torch.int32, (E,))
    _dev(gsum, "gsum", torch.float64, (E,))
    _dev(lse2sum, "lse2sum", torch.float64, (1,))
    if hsum is not None:
        _dev(hsum, "hsum", torch.float64, (1,))
    dev = n.device
    s = make_shape(T, 8, E, k, 8, dtype=torch.float32)
    out = {"f": torch.empty(E, dtype=torch.float32, device=dev),
           "P": torch.empty(E, dtype=torch.float32, device=dev),
           "aux": torch.empty(1, dtype=torch.float32, device=dev),
           "z": torch.empty(1, dtype=torch.float32, device=dev),
           "diag": None if hsum is None else torch.empty(4, dtype=torch.float32, device=dev),
           "b_new": None if b is None else torch.empty(E, dtype=torch.float32, device=dev)}
    if b is not None:
        _dev(b, "b", torch.float32, (E,))
    _check(lib().moe_balance_stats(ctypes.byref(s), _ptr(n), _ptr(gsum), _ptr(lse2sum), _ptr(hsum),
                                   float(lam), _ptr(out["f"]), _ptr(out["P"]), _ptr(out["aux"]),
                                   _ptr(out["z"]), _ptr(out["diag"]), _ptr(b), _ptr(out["b_new"]),
                                   float(gamma), _stream()),
           "moe_balance_stats")
    return out


def moe_balance_loss_backward(x: torch.Tensor, W_r: torch.Tensor, n: torch.Tensor, k: int,
                              lam: float = 0.01, z_coef: float = 1.0, c: Optional[float] = None,
                              scoring: str = "softmax", routing: str = "token",
                              want=("dlogits", "dW_r", "dx"), ws: Optional[torch.Tensor] = None) -> dict:
    """Gradients of aux + z_coef z with respect to the router logits, W_r and x (fp32), f fixed
    at the forward's loads n."""
    T, d = x.shape
    E = W_r.shape[0]
    s = make_shape(T, d, E, k, 8, c=c, dtype=x.dtype, scoring=scoring, routing=routing)
    _dev(x, "x")
    _dev(W_r, "W_r", x.dtype, (E, d))
    _dev(n, "n", torch.int32, (E,))
    dev = x.device
    out = {"dlogits": torch.empty(T, E, dtype=torch.float32, device=dev) if "dlogits" in want else None,
           "dW_r": torch.empty(E, d, dtype=torch.float32, device=dev) if "dW_r" in want else None,
           "dx": torch.empty(T, d, dtype=torch.float32, device=dev) if "dx" in want else None}
    if ws is None:
        ws = workspace(s, CALL_LOSS_BACKWARD, dev)
    _check(lib().moe_balance_loss_backward(ctypes.byref(s), _ptr(x), _ptr(W_r), _ptr(n), float(lam),
                                           float(z_coef), _ptr(out["dlogits"]), _ptr(out["dW_r"]),
                                           _ptr(out["dx"]), _ptr(ws), ws.numel(), _stream()),
           "moe_balance_loss_backward")
    return out


def saved_size(s: Shape) -> int:
    """moe_saved_size: bytes of the pre-activations a forward keeps for the backward (0: fp32)."""
    return int(lib().moe_saved_size(ctypes.byref(s)))


def saved_buffer(s: Shape, device) -> torch.Tensor:
    n = saved_size(s)
    if n == 0:
        raise ValueError("saved pre-activations are kept for bf16 layers only")
    return torch.empty(n, dtype=torch.uint8, device=device)


def _saved_ok(saved, s: Shape, dev) -> None:
    if saved.device != dev or not saved.is_contiguous() or saved.numel() < saved_size(s):
        raise ValueError("saved: a contiguous device buffer of saved_size(shape) bytes")


def moe_layer_backward(x, W_r, W_gate, W_up, W_down, dy, k: int, b=None, shared=None,
                       c: Optional[float] = None, renorm: bool = True, lam: float = 0.01,
                       z_coef: float = 0.0, scoring: str = "softmax", routing: str = "token",
                       ws: Optional[torch.Tensor] = None,
                       saved: Optional[torch.Tensor] = None) -> dict:
    """Gradients (fp32) of <dy, y> + aux + z_coef z for the layer; ``shared`` is the stacked
    (Ws_gate, Ws_up, Ws_down) when the layer has shared experts. ``topk_idx`` is the recomputed
    token-choice selection (left unwritten under expert choice). ``saved``: the buffer a forward
    on the same inputs filled (``MoELayer.forward(..., saved=...)``); the gate/up pre-activations
    are then taken from it instead of being recomputed (bf16 layers)."""
    T, d = x.shape
    E, M, _ = W_gate.shape
    S = _shared_count(shared, M, d, x.dtype)
    s = make_shape(T, d, E, k, M, S, c, renorm, x.dtype, scoring, routing)
    _check(check_shape(s), "moe_layer_backward")
    dt = x.dtype
    for name, t, shp in (("x", x, (T, d)), ("W_r", W_r, (E, d)), ("W_gate", W_gate, (E, M, d)),
                         ("W_up", W_up, (E, M, d)), ("W_down", W_down, (E, d, M)),
                         ("dy", dy, (T, d))):
        _dev(t, name, dt, shp)
    if b is not None:
        _dev(b, "b", torch.float32, (E,))
    dev = x.device
    f32 = dict(dtype=torch.float32, device=dev)
    out = {"dx": torch.empty(T, d, **f32), "dW_r": torch.empty(E, d, **f32),
           "dW_gate": torch.empty(E, M, d, **f32), "dW_up": torch.empty(E, M, d, **f32),
           "dW_down": torch.empty(E, d, M, **f32),
           "topk_idx": torch.empty(T, k, dtype=torch.int32, device=dev)}
    sg = su = sd = None
    if S > 0:
        sg, su, sd = shared
        out.update({"dWs_gate": torch.empty(S * M, d, **f32), "dWs_up": torch.empty(S * M, d, **f32),
                    "dWs_down": torch.empty(d, S * M, **f32)})
    if ws is None:
        ws = workspace(s, CALL_LAYER_BACKWARD, dev)
    if saved is not None:
        _saved_ok(saved, s, dev)
    _check(lib().moe_layer_backward(
        ctypes.byref(s), _ptr(x), _ptr(W_r), _ptr(b), _ptr(W_gate), _ptr(W_up), _ptr(W_down),
        _ptr(sg), _ptr(su), _ptr(sd), _ptr(dy), float(lam), float(z_coef), _ptr(out["dx"]),
        _ptr(out["dW_r"]), _ptr(out["dW_gate"]), _ptr(out["dW_up"]), _ptr(out["dW_down"]),
        _ptr(out.get("dWs_gate")), _ptr(out.get("dWs_up")), _ptr(out.get("dWs_down")),
        _ptr(out["topk_idx"]), _ptr(saved), _ptr(ws), ws.numel(), _stream()), "moe_layer_backward")
    return out


class MoELayer:
    """Holds the sizes and a preallocated workspace; ``forward`` calls moe_layer_forward, or, with
    ``noalloc=True``, moe_layer_forward_noalloc, which takes its workspace from the library's
    static scratch (construct with ``with_workspace=False`` and pass preallocated ``out`` tensors
    to allocate nothing at all)."""

    def __init__(self, T: int, d: int, E: int, k: int, M: int, S: int = 0,
                 c: Optional[float] = None, renorm: bool = True,
                 dtype: torch.dtype = torch.bfloat16, device="cuda", scoring: str = "softmax",
                 routing: str = "token", with_workspace: bool = True):
        self.shape = make_shape(T, d, E, k, M, S, c, renorm, dtype, scoring, routing)
        _check(check_shape(self.shape), "MoELayer")
        self.T, self.d, self.E, self.k, self.M, self.S = T, d, E, k, M, S
        self.dtype = dtype
        self.device = torch.device(device)
        self.ws = workspace(self.shape, CALL_LAYER, self.device) if with_workspace else None

    def alloc_outputs(self, with_bias: bool = False, placement: bool = False) -> dict:
        """Output tensors; ``placement`` adds inv_perm [T, k] (token choice) and perm_token
        [routed_rows] (the dispatch of "MoE：条件计算与路由" §3 the layer made)."""
        dev, T, E, k = self.device, self.T, self.E, self.k
        token = self.shape.routing == ROUTING["token"]
        return {"y": torch.empty(T, self.d, dtype=self.dtype, device=dev),
                "inv_perm": torch.empty(T, k, dtype=torch.int32, device=dev)
                if placement and token else None,
                "perm_token": torch.full((max(routed_rows(self.shape), 1),), -1, dtype=torch.int32,
                                         device=dev) if placement else None,
                "topk_idx": torch.empty(T, k, dtype=torch.int32, device=dev),
                "topk_w": torch.empty(T, k, dtype=torch.float32, device=dev),
                "counts": torch.empty(E, dtype=torch.int32, device=dev),
                "overflow": torch.empty(E, dtype=torch.int32, device=dev),
                "f": torch.empty(E, dtype=torch.float32, device=dev),
                "P": torch.empty(E, dtype=torch.float32, device=dev),
                "aux": torch.empty(1, dtype=torch.float32, device=dev),
                "z": torch.empty(1, dtype=torch.float32, device=dev),
                "diag": torch.empty(4, dtype=torch.float32, device=dev),
                "b_new": torch.empty(E, dtype=torch.float32, device=dev) if with_bias else None}

    def saved_buffer(self) -> torch.Tensor:
        """A buffer for ``forward(..., saved=...)`` (bf16 layers): moe_saved_size bytes."""
        return saved_buffer(self.shape, self.device)

    def forward(self, x, W_r, W_gate, W_up, W_down, b=None, shared=None, lam: float = 0.01,
                gamma: float = 1e-3, out: Optional[dict] = None,
                saved: Optional[torch.Tensor] = None, noalloc: bool = False) -> dict:
        T, d, E, M, dt = self.T, self.d, self.E, self.M, self.dtype
        _dev(x, "x", dt, (T, d))
        _dev(W_r, "W_r", dt, (E, d))
        _dev(W_gate, "W_gate", dt, (E, M, d))
        _dev(W_up, "W_up", dt, (E, M, d))
        _dev(W_down, "W_down", dt, (E, d, M))
        if b is not None:
            _dev(b, "b", torch.float32, (E,))
        sg = su = sd = None
        if self.S > 0:
            if shared is None:
                raise ValueError("this layer has shared experts: pass shared=(Ws_gate, Ws_up, Ws_down)")
            sg, su, sd = shared
            SM = self.S * M
            _dev(sg, "Ws_gate", dt, (SM, d))
            _dev(su, "Ws_up", dt, (SM, d))
            _dev(sd, "Ws_down", dt, (d, SM))
        if out is None:
            out = self.alloc_outputs(with_bias=b is not None)
        if saved is not None:
            _saved_ok(saved, self.shape, self.device)
        args = (ctypes.byref(self.shape), _ptr(x), _ptr(W_r), _ptr(b), _ptr(W_gate), _ptr(W_up),
                _ptr(W_down), _ptr(sg), _ptr(su), _ptr(sd), _ptr(out["y"]),
                _ptr(out.get("topk_idx")), _ptr(out.get("topk_w")), _ptr(out.get("counts")),
                _ptr(out.get("overflow")), _ptr(out.get("f")), _ptr(out.get("P")),
                _ptr(out.get("aux")), _ptr(out.get("z")), _ptr(out.get("diag")),
                _ptr(out.get("b_new") if b is not None else None), _ptr(out.get("inv_perm")),
                _ptr(out.get("perm_token")), float(lam), float(gamma), _ptr(saved))
        if noalloc:
            _check(lib().moe_layer_forward_noalloc(*args, _stream()), "moe_layer_forward_noalloc")
        else:
            if self.ws is None:
                raise ValueError("this layer has no workspace: pass noalloc=True")
            _check(lib().moe_layer_forward(*args, _ptr(self.ws), self.ws.numel(), _stream()),
                   "moe_layer_forward")
        return out


_stage_events_held = None  # the events the library records into, kept alive while it may


def moe_set_stage_events(events) -> None:
    """Profiling aid: record ``events`` (8 torch.cuda.Event, timing enabled) at the end of each
    stage of later moe_layer_forward calls; None switches recording off. The events are kept
    referenced here until recording is switched off."""
    global _stage_events_held
    if events is None:
        _check(lib().moe_set_stage_events(None, 0), "moe_set_stage_events")
        torch.cuda.synchronize()  # forwards already enqueued may still record into them
        _stage_events_held = None
        return
    arr = (ctypes.c_void_p * len(events))()
    stream = torch.cuda.current_stream()
    for i, ev in enumerate(events):
        if not ev.cuda_event:
            ev.record(stream)  # torch creates the HIP event on its first record
        arr[i] = ev.cuda_event
    _check(lib().moe_set_stage_events(arr, len(events)), "moe_set_stage_events")
    _stage_events_held = list(events)


def moe_layer_forward(x, W_r, W_gate, W_up, W_down, k: int, b=None, shared=None,
                      c: Optional[float] = None, renorm: bool = True, lam: float = 0.01,
                      gamma: float = 1e-3, scoring: str = "softmax", routing: str = "token") -> dict:
    """One call of the whole layer (allocates its workspace; use MoELayer to reuse one)."""
    T, d = x.shape
    E, M, _ = W_gate.shape
    S = _shared_count(shared, M, d, x.dtype)
    layer = MoELayer(T, d, E, k, M, S, c, renorm, x.dtype, x.device, scoring, routing)
    return layer.forward(x, W_r, W_gate, W_up, W_down, b, shared, lam, gamma)


__all__ = ["moe_route", "moe_dispatch", "moe_expert_ffn", "moe_combine", "moe_balance_stats",
           "moe_balance_loss_backward", "moe_layer_backward",
           "moe_layer_forward", "MoELayer", "make_shape", "capacity", "workspace_size",
           "check_shape", "status_string", "lib", "MoEError", "Shape", "moe_set_stage_events",
           "routed_rows", "saved_size"]

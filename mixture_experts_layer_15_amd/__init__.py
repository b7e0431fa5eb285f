"""MI355X (gfx950) sparse Mixture-of-Experts FFN forward.

A thin ctypes binding over libmoe_mi355x.so (C ABI: include/moe.h).  This
module only marshals arguments: it checks tensor dtypes, devices and shapes,
allocates outputs with torch (device memory is torch's), and passes raw
pointers and the current HIP stream.  Every step of the layer runs in the
library's HIP kernels; there is no fallback path, and a missing or unloadable
library raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Tuple

from .configs import CONFIGS, MoEConfig, get  # noqa: F401

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_mi355x.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
MOE_F32, MOE_BF16 = 0, 1
MOE_DROP_TOKEN_ORDER, MOE_DROP_CHOICE_ORDER = 0, 1
MOE_LAYOUT_COMPACT, MOE_LAYOUT_PADDED = 0, 1

EXPORTS = ("moe_capacity", "moe_max_rows", "moe_workspace_size", "moe_dispatch_workspace_size",
           "moe_status_string",
           "moe_last_error", "moe_route", "moe_route_from_logits", "moe_dispatch",
           "moe_dispatch_noalloc",
           "moe_expert_ffn", "moe_expert_gate_up", "moe_expert_down", "moe_combine",
           "moe_forward", "moe_load_stats", "moe_pid_update", "moe_mlp_router_workspace_size",
           "moe_route_mlp", "moe_backward_workspace_size", "moe_backward",
           # measurement probes (include/moe_probe.h)
           "moe_probe_copy", "moe_probe_read", "moe_probe_mfma")


class CConfig(ctypes.Structure):
    """Mirror of moe_config (include/moe.h)."""
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("temperature", ctypes.c_float), ("cap_num", ctypes.c_int32),
                ("cap_den", ctypes.c_int32), ("renormalize", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("drop_policy", ctypes.c_int32),
                ("layout", ctypes.c_int32), ("route_threshold", ctypes.c_float),
                ("k_min", ctypes.c_int32)]


class CMLPRouter(ctypes.Structure):
    """Mirror of moe_mlp_router (include/moe.h)."""
    _fields_ = [("r", ctypes.c_int32), ("m", ctypes.c_int32), ("gamma", ctypes.c_float),
                ("eps", ctypes.c_float), ("w_down", ctypes.c_void_p), ("b_down", ctypes.c_void_p),
                ("w1", ctypes.c_void_p), ("b1", ctypes.c_void_p), ("w2", ctypes.c_void_p),
                ("b2", ctypes.c_void_p), ("w3", ctypes.c_void_p), ("b3", ctypes.c_void_p),
                ("pid_bias", ctypes.c_void_p)]


class CPIDGains(ctypes.Structure):
    """Mirror of moe_pid_gains (include/moe.h)."""
    _fields_ = [("kp", ctypes.c_double), ("ki", ctypes.c_double), ("kd", ctypes.c_double),
                ("scale", ctypes.c_double)]


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        super().__init__(f"{where}: status {status} ({message})")
        self.status = status


_lib = None
_P = ctypes.c_void_p


def lib() -> ctypes.CDLL:
    """The loaded C library (raises if it was never built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} not found: build it first (python -m mixture_experts_layer_15_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        cp = ctypes.POINTER(CConfig)
        L.moe_capacity.argtypes = [cp]
        L.moe_capacity.restype = ctypes.c_int64
        L.moe_max_rows.argtypes = [cp]
        L.moe_max_rows.restype = ctypes.c_int64
        L.moe_workspace_size.argtypes = [cp, ctypes.POINTER(ctypes.c_size_t)]
        L.moe_workspace_size.restype = ctypes.c_int
        L.moe_dispatch_workspace_size.argtypes = [cp, ctypes.POINTER(ctypes.c_size_t)]
        L.moe_dispatch_workspace_size.restype = ctypes.c_int
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_last_error.argtypes = []
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_route.argtypes = [cp, _P, _P, _P, _P, _P, _P, _P]
        L.moe_route_from_logits.argtypes = [cp, _P, _P, _P, _P]
        L.moe_dispatch.argtypes = [cp, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.moe_dispatch_noalloc.argtypes = [cp, _P, _P, _P, _P, _P, _P, _P, _P]
        L.moe_expert_ffn.argtypes = [cp, _P, _P, _P, _P, _P, _P, _P, _P]
        L.moe_expert_gate_up.argtypes = [cp, _P, _P, _P, _P, _P, _P]
        L.moe_expert_down.argtypes = [cp, _P, _P, _P, _P, _P]
        L.moe_combine.argtypes = [cp, _P, _P, _P, _P, _P]
        L.moe_forward.argtypes = [cp, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.moe_load_stats.argtypes = [cp, _P, _P, _P]
        L.moe_pid_update.argtypes = [cp, ctypes.POINTER(CPIDGains), _P, _P, _P, _P]
        rp = ctypes.POINTER(CMLPRouter)
        L.moe_mlp_router_workspace_size.argtypes = [cp, rp, ctypes.POINTER(ctypes.c_size_t)]
        L.moe_route_mlp.argtypes = [cp, rp, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.moe_backward_workspace_size.argtypes = [cp, ctypes.POINTER(ctypes.c_size_t)]
        L.moe_backward.argtypes = [cp] + [_P] * 15 + [ctypes.c_size_t, _P]
        for n in ("moe_route", "moe_route_from_logits", "moe_dispatch", "moe_dispatch_noalloc",
                  "moe_expert_ffn",
                  "moe_expert_gate_up", "moe_expert_down", "moe_combine", "moe_forward",
                  "moe_load_stats", "moe_pid_update", "moe_mlp_router_workspace_size",
                  "moe_route_mlp",
                  "moe_backward_workspace_size", "moe_backward",
           # measurement probes (include/moe_probe.h)
           "moe_probe_copy", "moe_probe_read", "moe_probe_mfma"):
            getattr(L, n).restype = ctypes.c_int
        _lib = L
    return _lib


def cconfig(cfg: MoEConfig, T: Optional[int] = None) -> CConfig:
    return CConfig(T=cfg.T if T is None else T, d=cfg.d, E=cfg.E, k=cfg.k, d_ff=cfg.d_ff,
                   temperature=cfg.temperature, cap_num=cfg.cap_num, cap_den=cfg.cap_den,
                   renormalize=int(cfg.renormalize),
                   dtype=MOE_BF16 if cfg.dtype == "bf16" else MOE_F32,
                   drop_policy=int(cfg.drop_policy), layout=int(cfg.layout),
                   route_threshold=float(cfg.route_threshold), k_min=int(cfg.k_min))


def _check(status: int, where: str) -> None:
    if status != MOE_OK:
        msg = lib().moe_last_error().decode()
        raise MoEError(status, where, msg or lib().moe_status_string(status).decode())


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t) -> Optional[int]:
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtype, shape, device):
    import torch
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous() \
            or t.device != device:
        raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)} on {device}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}"
                         f"{'' if t.is_contiguous() else ' (not contiguous)'}")


# Output sentinels, off by default (tests turn them on): every output the
# binding allocates then starts as NaN (floating) or -7 (integer) and every
# workspace as 0xFF bytes, so an element that a kernel fails to write shows
# up in a comparison instead of passing on a stale value.
_SENTINELS = os.environ.get("MOE_OUTPUT_SENTINELS", "") == "1"


def set_output_sentinels(on: bool) -> None:
    global _SENTINELS
    _SENTINELS = bool(on)


def _out(shape, dtype, device):
    import torch
    shape = (shape,) if isinstance(shape, int) else tuple(shape)
    if not _SENTINELS:
        return torch.empty(shape, dtype=dtype, device=device)
    fill = float("nan") if dtype.is_floating_point else -7
    return torch.full(shape, fill, dtype=dtype, device=device)


def _workspace(nbytes: int, device):
    import torch
    n = max(int(nbytes), 16)
    if not _SENTINELS:
        return torch.empty(n, dtype=torch.uint8, device=device)
    return torch.full((n,), 0xFF, dtype=torch.uint8, device=device)


def _dt(cfg: MoEConfig):
    import torch
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def capacity(cfg: MoEConfig) -> int:
    return int(lib().moe_capacity(ctypes.byref(cconfig(cfg))))


def max_rows(cfg: MoEConfig) -> int:
    return int(lib().moe_max_rows(ctypes.byref(cconfig(cfg))))


def workspace_bytes(cfg: MoEConfig, dispatch_only: bool = False) -> int:
    """moe_workspace_size (moe_forward), or moe_dispatch_workspace_size."""
    n = ctypes.c_size_t(0)
    fn = lib().moe_dispatch_workspace_size if dispatch_only else lib().moe_workspace_size
    _check(fn(ctypes.byref(cconfig(cfg)), ctypes.byref(n)),
           "moe_dispatch_workspace_size" if dispatch_only else "moe_workspace_size")
    return n.value


def route(cfg: MoEConfig, x, w_router, bias=None):
    """moe_route -> (logits [T,E] fp32, topk_idx [T,k] int32, topk_gate [T,k] fp32)."""
    import torch
    dev = x.device
    _need(x, "x", _dt(cfg), (cfg.T, cfg.d), dev)
    _need(w_router, "w_router", _dt(cfg), (cfg.d, cfg.E), dev)
    if bias is not None:
        _need(bias, "bias", torch.float32, (cfg.E,), dev)
    logits = _out((cfg.T, cfg.E), torch.float32, dev)
    idx = _out((cfg.T, cfg.k), torch.int32, dev)
    gate = _out((cfg.T, cfg.k), torch.float32, dev)
    _check(lib().moe_route(ctypes.byref(cconfig(cfg)), _ptr(x), _ptr(w_router), _ptr(bias),
                           _ptr(logits), _ptr(idx), _ptr(gate), _stream()), "moe_route")
    return logits, idx, gate


def route_from_logits(cfg: MoEConfig, logits):
    """moe_route_from_logits -> (topk_idx, topk_gate) from given fp32 logits."""
    import torch
    dev = logits.device
    _need(logits, "logits", torch.float32, (cfg.T, cfg.E), dev)
    idx = _out((cfg.T, cfg.k), torch.int32, dev)
    gate = _out((cfg.T, cfg.k), torch.float32, dev)
    _check(lib().moe_route_from_logits(ctypes.byref(cconfig(cfg)), _ptr(logits), _ptr(idx),
                                       _ptr(gate), _stream()), "moe_route_from_logits")
    return idx, gate


def dispatch(cfg: MoEConfig, topk_idx, x) -> Dict:
    """moe_dispatch -> dict(x_perm, expert_count, expert_offset, row_of, token_of_row)."""
    import torch
    dev = x.device
    _need(topk_idx, "topk_idx", torch.int32, (cfg.T, cfg.k), dev)
    _need(x, "x", _dt(cfg), (cfg.T, cfg.d), dev)
    R = max_rows(cfg)
    out = dict(
        x_perm=_out((R, cfg.d), _dt(cfg), dev),
        expert_count=_out(cfg.E, torch.int32, dev),
        expert_offset=_out(cfg.E + 1, torch.int32, dev),
        row_of=_out((cfg.T, cfg.k), torch.int32, dev),
        token_of_row=_out(max(cfg.T * cfg.k, R), torch.int32, dev))
    wsb = workspace_bytes(cfg, dispatch_only=True)
    ws = _workspace(wsb, dev)
    _check(lib().moe_dispatch(ctypes.byref(cconfig(cfg)), _ptr(topk_idx), _ptr(x),
                              _ptr(out["x_perm"]), _ptr(out["expert_count"]),
                              _ptr(out["expert_offset"]), _ptr(out["row_of"]),
                              _ptr(out["token_of_row"]), _ptr(ws), wsb, _stream()),
           "moe_dispatch")
    out["_workspace"] = ws   # keep alive until the stream has run
    return out


MLP_ROUTER_KEYS = ("w_down", "b_down", "w1", "b1", "w2", "b2", "w3", "b3", "pid_bias")


def route_mlp(cfg: MoEConfig, x, prev, router: Dict, gamma: float, eps: float):
    """moe_route_mlp -> (logits [T,E] fp32, topk_idx [T,k] int32, topk_gate [T,k] fp32).
    router: dict of the weights (w_down [d,r], w1 [r,m], w2 [m,m], w3 [m,E], layer dtype)
    and optional fp32 biases (b_down, b1, b2, b3, pid_bias)."""
    import torch
    dev = x.device
    r, m = router["w_down"].shape[1], router["w1"].shape[1]
    _need(x, "x", _dt(cfg), (cfg.T, cfg.d), dev)
    if prev is not None:
        _need(prev, "prev", _dt(cfg), (cfg.T, r), dev)
    for key, shape in (("w_down", (cfg.d, r)), ("w1", (r, m)), ("w2", (m, m)), ("w3", (m, cfg.E))):
        _need(router[key], key, _dt(cfg), shape, dev)
    for key, n in (("b_down", r), ("b1", m), ("b2", m), ("b3", cfg.E), ("pid_bias", cfg.E)):
        if router.get(key) is not None:
            _need(router[key], key, torch.float32, (n,), dev)
    addr = lambda t: None if t is None else t.data_ptr()
    cr = CMLPRouter(r=r, m=m, gamma=gamma, eps=eps,
                    **{key: addr(router.get(key)) for key in MLP_ROUTER_KEYS})
    c = cconfig(cfg)
    n = ctypes.c_size_t(0)
    _check(lib().moe_mlp_router_workspace_size(ctypes.byref(c), ctypes.byref(cr), ctypes.byref(n)),
           "moe_mlp_router_workspace_size")
    ws = _workspace(n.value, dev)
    logits = _out((cfg.T, cfg.E), torch.float32, dev)
    idx = _out((cfg.T, cfg.k), torch.int32, dev)
    gate = _out((cfg.T, cfg.k), torch.float32, dev)
    _check(lib().moe_route_mlp(ctypes.byref(c), ctypes.byref(cr), _ptr(x), _ptr(prev),
                               _ptr(logits), _ptr(idx), _ptr(gate), _ptr(ws), n.value, _stream()),
           "moe_route_mlp")
    route_mlp._last_ws = ws   # keep the workspace alive until the stream has run
    return logits, idx, gate


def load_stats(cfg: MoEConfig, expert_count):
    """moe_load_stats -> fp64 [8]: mean, max, min, max/mean, max |count - mean| / mean,
    std / mean, dropped assignments, empty experts (counts before drops)."""
    import torch
    dev = expert_count.device
    _need(expert_count, "expert_count", torch.int32, (cfg.E,), dev)
    stats = _out(8, torch.float64, dev)
    _check(lib().moe_load_stats(ctypes.byref(cconfig(cfg)), _ptr(expert_count), _ptr(stats),
                                _stream()), "moe_load_stats")
    return stats


def pid_update(cfg: MoEConfig, expert_count, state, kp: float, ki: float, kd: float,
               scale: float = 1.0):
    """moe_pid_update: one step of the load-balance PID controller.  state
    [2, E] fp64 (integrals, previous errors) is updated in place; returns the
    logit bias pid_bias [E] fp32."""
    import torch
    dev = expert_count.device
    _need(expert_count, "expert_count", torch.int32, (cfg.E,), dev)
    _need(state, "state", torch.float64, (2, cfg.E), dev)
    bias = _out(cfg.E, torch.float32, dev)
    g = CPIDGains(kp=float(kp), ki=float(ki), kd=float(kd), scale=float(scale))
    _check(lib().moe_pid_update(ctypes.byref(cconfig(cfg)), ctypes.byref(g), _ptr(expert_count),
                                _ptr(state), _ptr(bias), _stream()), "moe_pid_update")
    return bias


def expert_ffn(cfg: MoEConfig, x_perm, expert_offset, w_gate, w_up, w_down) -> Tuple:
    """moe_expert_ffn -> (h [R, d_ff], y_perm [R, d])."""
    import torch
    dev = x_perm.device
    R = max_rows(cfg)
    _need(x_perm, "x_perm", _dt(cfg), (R, cfg.d), dev)
    _need(expert_offset, "expert_offset", torch.int32, (cfg.E + 1,), dev)
    _need(w_gate, "w_gate", _dt(cfg), (cfg.E, cfg.d, cfg.d_ff), dev)
    _need(w_up, "w_up", _dt(cfg), (cfg.E, cfg.d, cfg.d_ff), dev)
    _need(w_down, "w_down", _dt(cfg), (cfg.E, cfg.d_ff, cfg.d), dev)
    h = _out((R, cfg.d_ff), _dt(cfg), dev)
    y_perm = _out((R, cfg.d), _dt(cfg), dev)
    _check(lib().moe_expert_ffn(ctypes.byref(cconfig(cfg)), _ptr(x_perm), _ptr(expert_offset),
                                _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(h), _ptr(y_perm),
                                _stream()), "moe_expert_ffn")
    return h, y_perm


def expert_gate_up(cfg: MoEConfig, x_perm, expert_offset, w_gate, w_up, h=None):
    """moe_expert_gate_up -> h [R, d_ff]."""
    import torch
    dev = x_perm.device
    R = max_rows(cfg)
    _need(x_perm, "x_perm", _dt(cfg), (R, cfg.d), dev)
    _need(expert_offset, "expert_offset", torch.int32, (cfg.E + 1,), dev)
    _need(w_gate, "w_gate", _dt(cfg), (cfg.E, cfg.d, cfg.d_ff), dev)
    _need(w_up, "w_up", _dt(cfg), (cfg.E, cfg.d, cfg.d_ff), dev)
    if h is None:
        h = _out((R, cfg.d_ff), _dt(cfg), dev)
    _need(h, "h", _dt(cfg), (R, cfg.d_ff), dev)
    _check(lib().moe_expert_gate_up(ctypes.byref(cconfig(cfg)), _ptr(x_perm), _ptr(expert_offset),
                                    _ptr(w_gate), _ptr(w_up), _ptr(h), _stream()),
           "moe_expert_gate_up")
    return h


def expert_down(cfg: MoEConfig, h, expert_offset, w_down, y_perm=None):
    """moe_expert_down -> y_perm [R, d]."""
    import torch
    dev = h.device
    R = max_rows(cfg)
    _need(h, "h", _dt(cfg), (R, cfg.d_ff), dev)
    _need(expert_offset, "expert_offset", torch.int32, (cfg.E + 1,), dev)
    _need(w_down, "w_down", _dt(cfg), (cfg.E, cfg.d_ff, cfg.d), dev)
    if y_perm is None:
        y_perm = _out((R, cfg.d), _dt(cfg), dev)
    _need(y_perm, "y_perm", _dt(cfg), (R, cfg.d), dev)
    _check(lib().moe_expert_down(ctypes.byref(cconfig(cfg)), _ptr(h), _ptr(expert_offset),
                                 _ptr(w_down), _ptr(y_perm), _stream()), "moe_expert_down")
    return y_perm


def combine(cfg: MoEConfig, y_perm, row_of, topk_gate):
    """moe_combine -> y [T, d]."""
    import torch
    dev = y_perm.device
    _need(y_perm, "y_perm", _dt(cfg), (max_rows(cfg), cfg.d), dev)
    _need(row_of, "row_of", torch.int32, (cfg.T, cfg.k), dev)
    _need(topk_gate, "topk_gate", torch.float32, (cfg.T, cfg.k), dev)
    y = _out((cfg.T, cfg.d), _dt(cfg), dev)
    _check(lib().moe_combine(ctypes.byref(cconfig(cfg)), _ptr(y_perm), _ptr(row_of),
                             _ptr(topk_gate), _ptr(y), _stream()), "moe_combine")
    return y


class Forward:
    """moe_forward with a workspace allocated once and reused across calls."""

    def __init__(self, cfg: MoEConfig, device="cuda"):
        import torch
        self.cfg = cfg
        self.c = cconfig(cfg)
        self.ws_bytes = workspace_bytes(cfg)
        self.ws = _workspace(self.ws_bytes, device)

    def __call__(self, x, w_router, bias, w_gate, w_up, w_down, y=None):
        import torch
        cfg = self.cfg
        dev = x.device
        _need(x, "x", _dt(cfg), (cfg.T, cfg.d), dev)
        _need(w_router, "w_router", _dt(cfg), (cfg.d, cfg.E), dev)
        if bias is not None:
            _need(bias, "bias", torch.float32, (cfg.E,), dev)
        _need(w_gate, "w_gate", _dt(cfg), (cfg.E, cfg.d, cfg.d_ff), dev)
        _need(w_up, "w_up", _dt(cfg), (cfg.E, cfg.d, cfg.d_ff), dev)
        _need(w_down, "w_down", _dt(cfg), (cfg.E, cfg.d_ff, cfg.d), dev)
        if y is None:
            y = _out((cfg.T, cfg.d), _dt(cfg), dev)
        if _SENTINELS:   # no call may depend on what an earlier one left behind
            self.ws.fill_(0xFF)
        _check(lib().moe_forward(ctypes.byref(self.c), _ptr(x), _ptr(w_router), _ptr(bias),
                                 _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(y), _ptr(self.ws),
                                 self.ws_bytes, _stream()), "moe_forward")
        return y


def forward(cfg: MoEConfig, x, w_router, bias, w_gate, w_up, w_down):
    """moe_forward -> y [T, d] (allocates a fresh workspace)."""
    return Forward(cfg, device=x.device)(x, w_router, bias, w_gate, w_up, w_down)


def backward_workspace_bytes(cfg: MoEConfig) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_backward_workspace_size(ctypes.byref(cconfig(cfg)), ctypes.byref(n)),
           "moe_backward_workspace_size")
    return int(n.value)


class Backward:
    """moe_backward with a workspace allocated once and reused across calls."""

    def __init__(self, cfg: MoEConfig, device="cuda"):
        import torch
        self.cfg = cfg
        self.c = cconfig(cfg)
        self.ws_bytes = backward_workspace_bytes(cfg)
        self.ws = _workspace(self.ws_bytes, device)

    def __call__(self, x, w_router, bias, w_gate, w_up, w_down, dy, out: Optional[Dict] = None,
                 want_dgate: bool = True, want_dbias: bool = True) -> Dict:
        """Gradients dx (layer dtype), dw_router, dbias, dw_gate, dw_up, dw_down and
        dgate (fp32); ``out`` may hold preallocated tensors under those names."""
        import torch
        cfg = self.cfg
        dev = x.device
        dt = _dt(cfg)
        _need(x, "x", dt, (cfg.T, cfg.d), dev)
        _need(w_router, "w_router", dt, (cfg.d, cfg.E), dev)
        if bias is not None:
            _need(bias, "bias", torch.float32, (cfg.E,), dev)
        _need(w_gate, "w_gate", dt, (cfg.E, cfg.d, cfg.d_ff), dev)
        _need(w_up, "w_up", dt, (cfg.E, cfg.d, cfg.d_ff), dev)
        _need(w_down, "w_down", dt, (cfg.E, cfg.d_ff, cfg.d), dev)
        _need(dy, "dy", dt, (cfg.T, cfg.d), dev)
        shapes = dict(dx=((cfg.T, cfg.d), dt), dw_router=((cfg.d, cfg.E), torch.float32),
                      dbias=((cfg.E,), torch.float32),
                      dw_gate=((cfg.E, cfg.d, cfg.d_ff), torch.float32),
                      dw_up=((cfg.E, cfg.d, cfg.d_ff), torch.float32),
                      dw_down=((cfg.E, cfg.d_ff, cfg.d), torch.float32),
                      dgate=((cfg.T, cfg.k), torch.float32))
        g = dict(out or {})
        for name, (shape, tdt) in shapes.items():
            if (name == "dgate" and not want_dgate) or (name == "dbias" and not want_dbias):
                g[name] = None
                continue
            if g.get(name) is None:
                g[name] = _out(shape, tdt, dev)
            _need(g[name], name, tdt, shape, dev)
        if _SENTINELS:
            self.ws.fill_(0xFF)
        _check(lib().moe_backward(ctypes.byref(self.c), _ptr(x), _ptr(w_router), _ptr(bias),
                                  _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(dy), _ptr(g["dx"]),
                                  _ptr(g["dw_router"]), _ptr(g["dbias"]), _ptr(g["dw_gate"]),
                                  _ptr(g["dw_up"]), _ptr(g["dw_down"]), _ptr(g["dgate"]),
                                  _ptr(self.ws), self.ws_bytes, _stream()), "moe_backward")
        return g


def backward(cfg: MoEConfig, x, w_router, bias, w_gate, w_up, w_down, dy) -> Dict:
    """moe_backward -> dict of gradients (allocates a fresh workspace)."""
    return Backward(cfg, device=x.device)(x, w_router, bias, w_gate, w_up, w_down, dy)

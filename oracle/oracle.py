"""Python front end of the fp64 CPU oracle (moe_oracle.c).

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this module.  It never imports the
HIP library or its binding, and the HIP library never imports it.

Arrays are passed as numpy arrays or CPU torch tensors: fp32 values, or bf16
values (torch.bfloat16, or their raw 16-bit patterns as uint16/int16).  All
arithmetic happens in fp64 in the C library; this file only moves arrays and
strings the C steps together in the order the layer defines them:
logits -> top-k and gates -> capacity -> token-order dispatch -> GeGLU expert
FFN per kept row -> gate-weighted combine.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")
# A different build of moe_oracle.c (the mutation tests plant mistakes in a
# copy of the source and check that the pins catch them).
_LIB_OVERRIDE = os.environ.get("MOE_ORACLE_LIB")
_lock = threading.Lock()
_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64


def build() -> str:
    """Compile moe_oracle.c with gcc (OpenMP, no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-std=c11", _SRC, "-o", _LIB + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None and _LIB_OVERRIDE:
            _lib = _declare(ctypes.CDLL(_LIB_OVERRIDE))
        if _lib is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
            _lib = _declare(ctypes.CDLL(_LIB))
    return _lib


def _declare(lib):
    lib.orc_logits.argtypes = [_I64, _I64, _I64, ctypes.c_int, _P, _P, _P, _P]
    lib.orc_logits.restype = None
    lib.orc_route.argtypes = [_I64, _I64, _I64, ctypes.c_double, ctypes.c_int, _P, _P, _P]
    lib.orc_route.restype = None
    lib.orc_capacity.argtypes = [_I64, _I64, _I64, _I64, _I64]
    lib.orc_capacity.restype = _I64
    lib.orc_dispatch.argtypes = [_I64, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, ctypes.c_int,
                                 ctypes.c_int]
    lib.orc_dispatch.restype = None
    lib.orc_load_stats.argtypes = [_I64, _P, _I64, _P]
    lib.orc_load_stats.restype = None
    lib.orc_pid_update.argtypes = [_I64] + [ctypes.c_double] * 4 + [_P, _P, _P]
    lib.orc_pid_update.restype = None
    lib.orc_mlp_router.argtypes = [_I64, _I64, _I64, _I64, _I64, ctypes.c_int, _P, _P,
                                   ctypes.c_double, ctypes.c_double] + [_P] * 13
    lib.orc_mlp_router.restype = None
    lib.orc_backward.argtypes = [_I64, _I64, _I64, _I64, _I64, ctypes.c_int, ctypes.c_double,
                                 ctypes.c_int] + [_P] * 17
    lib.orc_backward.restype = None
    lib.orc_backward_wentries.argtypes = [_I64, _I64, _I64, _I64, ctypes.c_int] + [_P] * 8 + \
        [_I64] + [_P] * 5
    lib.orc_backward_wentries.restype = None
    lib.orc_ffn_rows.argtypes = [_I64, _P, _P, _I64, _I64, ctypes.c_int,
                                 _P, _P, _P, _P, _P, _P]
    lib.orc_ffn_rows.restype = None
    lib.orc_combine.argtypes = [_I64, _P, _I64, _I64, _P, _P, _P, _P]
    lib.orc_combine.restype = None
    lib.orc_router_backward.argtypes = [_I64, _I64, _I64, ctypes.c_double, ctypes.c_int,
                                        _P, _P, _P, _P, _P]
    lib.orc_router_backward.restype = None
    lib.orc_route_dynamic.argtypes = [_I64, _I64, _I64, _I64, ctypes.c_double, ctypes.c_double,
                                      ctypes.c_int, _P, _P, _P]
    lib.orc_route_dynamic.restype = None
    lib.orc_capacity_realised.argtypes = [_I64, _I64, _I64, _I64, _I64]
    lib.orc_capacity_realised.restype = _I64
    return lib


def _raw(a):
    """numpy view of an input array, plus its dtype code (0 fp32, 1 bf16)."""
    if a is None:
        return None, None
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().cpu().contiguous()
            if a.dtype == torch.bfloat16:
                a = a.view(torch.int16).numpy().view(np.uint16)
            else:
                a = a.numpy()
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a, 0
    if a.dtype in (np.uint16, np.int16):
        return a.view(np.uint16), 1
    raise TypeError(f"oracle inputs must be fp32 or bf16, got {a.dtype}")


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def logits(x, w_router, bias=None) -> np.ndarray:
    """l[t][e] = sum_i x[t][i] Wr[i][e] + b[e], in fp64."""
    xr, dt = _raw(x)
    wr, dt2 = _raw(w_router)
    assert dt == dt2
    T, d = xr.shape
    E = wr.shape[1]
    b = None if bias is None else np.ascontiguousarray(_raw(bias)[0], dtype=np.float32)
    out = np.empty((T, E), dtype=np.float64)
    _load().orc_logits(T, d, E, dt, _ptr(xr), _ptr(wr), _ptr(b), _ptr(out))
    return out


def route(logits_, k: int, tau: float, renormalize: bool, k_min: int = 0,
          threshold: float = 0.0):
    """Top-k experts (logit descending, lower index on ties) and fp64 gates.
    threshold > 0: dynamic count per token (k_min .. k experts, the fewest
    whose softmax mass reaches threshold); unused slots hold -1 and gate 0."""
    lg = np.ascontiguousarray(logits_, dtype=np.float64)
    T, E = lg.shape
    idx = np.empty((T, k), dtype=np.int32)
    gate = np.empty((T, k), dtype=np.float64)
    if threshold > 0:
        _load().orc_route_dynamic(T, E, k, int(k_min), float(threshold), float(tau),
                                  int(bool(renormalize)), _ptr(lg), _ptr(idx), _ptr(gate))
    else:
        _load().orc_route(T, E, k, float(tau), int(bool(renormalize)), _ptr(lg), _ptr(idx),
                          _ptr(gate))
    return idx, gate


def capacity(T: int, E: int, k: int, cap_num: int, cap_den: int) -> int:
    return int(_load().orc_capacity(T, E, k, cap_num, cap_den))


def capacity_realised(idx: np.ndarray, E: int, cap_num: int, cap_den: int) -> int:
    """Capacity of a dynamically routed batch: from the realised number of
    assignments (slots of idx that are not -1)."""
    idx = np.asarray(idx)
    A = int((idx >= 0).sum())
    return int(_load().orc_capacity_realised(A, idx.shape[0], E, cap_num, cap_den))


def dispatch(idx: np.ndarray, E: int, C: int, policy: int = 0,
             layout: int = 0) -> Dict[str, np.ndarray]:
    """Positions in priority order (0: token order, 1: choice order), drops,
    counts, offsets and the permutation maps, in the compact layout (0) or
    padded to C rows per expert (1, empty rows marked -1 in token_of_row).
    n_kept = rows holding a token, n_rows = rows of the layout (offset[E])."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T, k = idx.shape
    count = np.empty(E, dtype=np.int32)
    kept = np.empty(E, dtype=np.int32)
    offset = np.empty(E + 1, dtype=np.int32)
    pos = np.empty((T, k), dtype=np.int32)
    row_of = np.empty((T, k), dtype=np.int32)
    token_of_row = np.full(max(T * k, E * C if layout == 1 else 0), -1, dtype=np.int32)
    _load().orc_dispatch(T, E, k, C, _ptr(idx), _ptr(count), _ptr(kept), _ptr(offset),
                         _ptr(pos), _ptr(row_of), _ptr(token_of_row), int(policy), int(layout))
    n_rows = int(offset[E])
    return dict(count=count, kept=kept, offset=offset, pos=pos, row_of=row_of,
                token_of_row=token_of_row[:n_rows].copy(), n_kept=int(kept.sum()),
                n_rows=n_rows)


def ffn_rows(tokens: Sequence[int], experts: Sequence[int], x, w_gate, w_up, w_down,
             want_h: bool = False):
    """GeGLU expert FFN, fp64, for each listed (token, expert) row."""
    xr, dt = _raw(x)
    wg, d1 = _raw(w_gate)
    wu, d2 = _raw(w_up)
    wd, d3 = _raw(w_down)
    assert dt == d1 == d2 == d3
    d = xr.shape[1]
    d_ff = wg.shape[2]
    tok = np.ascontiguousarray(tokens, dtype=np.int64)
    ex = np.ascontiguousarray(experts, dtype=np.int32)
    n = tok.shape[0]
    o = np.empty((n, d), dtype=np.float64)
    h = np.empty((n, d_ff), dtype=np.float64) if want_h else None
    if n:
        _load().orc_ffn_rows(n, _ptr(tok), _ptr(ex), d, d_ff, dt, _ptr(xr), _ptr(wg),
                             _ptr(wu), _ptr(wd), _ptr(h), _ptr(o))
    return (h, o) if want_h else o


def combine(tokens: Sequence[int], row_of: np.ndarray, gate: np.ndarray,
            o_slots: np.ndarray) -> np.ndarray:
    """y[t] = sum of gate * o over the kept assignments of each listed token.

    ``o_slots`` holds one row per (listed token, j): shape [n_tok * k, d]."""
    row_of = np.ascontiguousarray(row_of, dtype=np.int32)
    gate = np.ascontiguousarray(gate, dtype=np.float64)
    o_slots = np.ascontiguousarray(o_slots, dtype=np.float64)
    toks = np.ascontiguousarray(tokens, dtype=np.int64)
    k = row_of.shape[1]
    d = o_slots.shape[1]
    y = np.empty((toks.shape[0], d), dtype=np.float64)
    if toks.shape[0]:
        _load().orc_combine(toks.shape[0], _ptr(toks), k, d, _ptr(row_of), _ptr(gate),
                            _ptr(o_slots), _ptr(y))
    return y


def _f32_or_none(b):
    return None if b is None else np.ascontiguousarray(_raw(b)[0], dtype=np.float32)


def mlp_router(x, prev, gamma: float, eps: float, wd, bd, w1, b1, w2, b2, w3, b3, pid,
               want_hidden: bool = False) -> Dict[str, np.ndarray]:
    """The MLP router's logits (and, if asked, z, h1, h2) in fp64; inputs as
    torch tensors of one dtype (bf16 or fp32), biases fp32 or None."""
    xr, dt = _raw(x)
    T, d = xr.shape
    wdr, _ = _raw(wd)
    w1r, _ = _raw(w1)
    w2r, _ = _raw(w2)
    w3r, _ = _raw(w3)
    r, m, E = wdr.shape[1], w1r.shape[1], w3r.shape[1]
    prr = None if prev is None else _raw(prev)[0]
    bs = [_f32_or_none(b) for b in (bd, b1, b2, b3, pid)]
    lg = np.empty((T, E), dtype=np.float64)
    z = np.empty((T, r)) if want_hidden else None
    h1 = np.empty((T, m)) if want_hidden else None
    h2 = np.empty((T, m)) if want_hidden else None
    _load().orc_mlp_router(T, d, r, m, E, dt, _ptr(xr), _ptr(prr), float(gamma), float(eps),
                           _ptr(wdr), _ptr(bs[0]), _ptr(w1r), _ptr(bs[1]), _ptr(w2r), _ptr(bs[2]),
                           _ptr(w3r), _ptr(bs[3]), _ptr(bs[4]), _ptr(lg), _ptr(z), _ptr(h1),
                           _ptr(h2))
    return dict(logits=lg, z=z, h1=h1, h2=h2)


def backward(x, w_router, bias, w_gate, w_up, w_down, dy, *, k: int, tau: float,
             renormalize: bool, cap_num: int, cap_den: int, drop_policy: int = 0,
             logits_in: Optional[np.ndarray] = None,
             tokens: Optional[Sequence[int]] = None, k_min: int = 0,
             threshold: float = 0.0) -> Dict[str, np.ndarray]:
    """Gradients of the layer for an upstream dy [T, d] (fp64 or castable), in
    fp64: dx, dw_router, dbias, dw_gate, dw_up, dw_down, dgate, plus the routing
    they used.  Routing as in forward() (also the dynamic count, threshold > 0,
    whose unused slots carry no gradient): from logits_in when given.

    ``tokens`` limits the computation to the listed tokens (routing, capacity
    and dispatch still cover the whole batch): only dx and dgate are returned,
    one row per listed token -- they depend on nothing but that token's own
    routing, inputs and upstream gradient."""
    xr, dt = _raw(x)
    T, d = xr.shape
    wrr, _ = _raw(w_router)
    E = wrr.shape[1]
    wgr, _ = _raw(w_gate)
    wur, _ = _raw(w_up)
    wdr, _ = _raw(w_down)
    d_ff = wgr.shape[2]
    lg = logits(x, w_router, bias) if logits_in is None else np.asarray(logits_in, np.float64)
    lg = np.ascontiguousarray(lg)
    idx, gate = route(lg, k, tau, renormalize, k_min, threshold)
    C = capacity_realised(idx, E, cap_num, cap_den) if threshold > 0 else \
        capacity(T, E, k, cap_num, cap_den)
    dsp = dispatch(idx, E, C, drop_policy)
    dyr = np.ascontiguousarray(np.asarray(dy, dtype=np.float64))
    row_of = dsp["row_of"]
    if tokens is not None:
        toks = np.asarray(tokens, dtype=np.int64)
        n = toks.shape[0]
        sub = lambda a: np.ascontiguousarray(a[toks])
        out = dict(dx=np.empty((n, d)), dgate=np.empty((n, k)))
        _load().orc_backward(n, d, E, k, d_ff, dt, float(tau), int(bool(renormalize)),
                             _ptr(sub(xr)), _ptr(wrr), _ptr(sub(lg)), _ptr(sub(idx)),
                             _ptr(sub(gate)), _ptr(sub(row_of)), _ptr(wgr), _ptr(wur), _ptr(wdr),
                             _ptr(sub(dyr)), _ptr(out["dx"]), None, None, None, None, None,
                             _ptr(out["dgate"]))
        out.update(logits=lg, idx=idx, gate=gate, row_of=row_of, C=C, tokens=toks)
        return out
    out = dict(dx=np.empty((T, d)), dw_router=np.empty((d, E)), dbias=np.empty(E),
               dw_gate=np.empty((E, d, d_ff)), dw_up=np.empty((E, d, d_ff)),
               dw_down=np.empty((E, d_ff, d)), dgate=np.empty((T, k)))
    _load().orc_backward(T, d, E, k, d_ff, dt, float(tau), int(bool(renormalize)), _ptr(xr),
                         _ptr(wrr), _ptr(lg), _ptr(idx), _ptr(np.ascontiguousarray(gate)),
                         _ptr(row_of), _ptr(wgr), _ptr(wur), _ptr(wdr), _ptr(dyr),
                         _ptr(out["dx"]), _ptr(out["dw_router"]), _ptr(out["dbias"]),
                         _ptr(out["dw_gate"]), _ptr(out["dw_up"]), _ptr(out["dw_down"]),
                         _ptr(out["dgate"]))
    out.update(logits=lg, idx=idx, gate=gate, row_of=row_of, C=C)
    return out


def router_backward(logits_, idx, gate, dgate, tau: float, renormalize: bool) -> np.ndarray:
    """dlogit [T, E] from the gate gradients dgate [T, k] (0 where dropped):
    through the renormalised (or raw) gates and the temperature softmax."""
    lg = np.ascontiguousarray(logits_, dtype=np.float64)
    T, E = lg.shape
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    k = idx.shape[1]
    dl = np.empty((T, E), dtype=np.float64)
    _load().orc_router_backward(T, E, k, float(tau), int(bool(renormalize)), _ptr(lg), _ptr(idx),
                                _ptr(np.ascontiguousarray(gate, dtype=np.float64)),
                                _ptr(np.ascontiguousarray(dgate, dtype=np.float64)), _ptr(dl))
    return dl


WGRAD = {"dw_gate": 0, "dw_up": 1, "dw_down": 2}


def backward_weight_entries(x, w_gate, w_up, w_down, dy, idx, gate, row_of,
                            entries: Sequence[Tuple[str, int, int, int]]) -> np.ndarray:
    """Single entries (name, e, a, b) of dw_gate [E, d, d_ff], dw_up or
    dw_down [E, d_ff, d], each summed from its definition over the kept rows
    of expert e (routing idx, gate, row_of as returned by backward/forward)."""
    xr, dt = _raw(x)
    T, d = xr.shape
    wgr, _ = _raw(w_gate)
    wur, _ = _raw(w_up)
    wdr, _ = _raw(w_down)
    d_ff = wgr.shape[2]
    k = np.asarray(idx).shape[1]
    which = np.array([WGRAD[n] for n, _, _, _ in entries], dtype=np.int64)
    ee = np.array([e for _, e, _, _ in entries], dtype=np.int64)
    aa = np.array([a for _, _, a, _ in entries], dtype=np.int64)
    bb = np.array([b for _, _, _, b in entries], dtype=np.int64)
    out = np.empty(len(entries))
    _load().orc_backward_wentries(
        T, d, k, d_ff, dt, _ptr(xr), _ptr(np.ascontiguousarray(idx, dtype=np.int32)),
        _ptr(np.ascontiguousarray(gate, dtype=np.float64)),
        _ptr(np.ascontiguousarray(row_of, dtype=np.int32)), _ptr(wgr), _ptr(wur), _ptr(wdr),
        _ptr(np.ascontiguousarray(np.asarray(dy, dtype=np.float64))), len(entries), _ptr(which),
        _ptr(ee), _ptr(aa), _ptr(bb), _ptr(out))
    return out


def load_stats(count: np.ndarray, C: int) -> np.ndarray:
    """Expert-load telemetry (8 values, see orc_load_stats) from counts before drops."""
    count = np.ascontiguousarray(count, dtype=np.int32)
    out = np.empty(8, dtype=np.float64)
    _load().orc_load_stats(count.shape[0], _ptr(count), int(C), _ptr(out))
    return out


def pid_update(count: np.ndarray, state: np.ndarray, kp: float, ki: float, kd: float,
               scale: float = 1.0):
    """One step of the load-balance PID controller (see orc_pid_update):
    returns (new state [2, E], bias [E]) in fp64; the input state is not
    modified."""
    count = np.ascontiguousarray(count, dtype=np.int32)
    E = count.shape[0]
    st = np.array(state, dtype=np.float64, copy=True).reshape(2, E)
    st = np.ascontiguousarray(st)
    bias = np.empty(E, dtype=np.float64)
    _load().orc_pid_update(E, float(kp), float(ki), float(kd), float(scale), _ptr(count),
                           _ptr(st), _ptr(bias))
    return st, bias


def forward(x, w_router, bias, w_gate, w_up, w_down, *, k: int, tau: float,
            renormalize: bool, cap_num: int, cap_den: int, drop_policy: int = 0,
            logits_in: Optional[np.ndarray] = None,
            tokens: Optional[Sequence[int]] = None, want_h: bool = False,
            k_min: int = 0, threshold: float = 0.0) -> Dict:
    """The whole layer in fp64.

    ``logits_in`` replaces step 1 (routing then runs on exactly those values,
    e.g. fp32 logits exported by another implementation).  ``tokens`` limits
    the expert FFN and the combine to the listed tokens (routing, capacity and
    dispatch always cover the whole batch, since drops depend on every earlier
    token).  Returns every intermediate."""
    xr, _ = _raw(x)
    T = xr.shape[0]
    E = _raw(w_router)[0].shape[1]
    lg = logits(x, w_router, bias) if logits_in is None else np.asarray(logits_in, np.float64)
    idx, gate = route(lg, k, tau, renormalize, k_min, threshold)
    C = capacity_realised(idx, E, cap_num, cap_den) if threshold > 0 else \
        capacity(T, E, k, cap_num, cap_den)
    dsp = dispatch(idx, E, C, drop_policy)
    toks = np.arange(T, dtype=np.int64) if tokens is None else np.asarray(tokens, np.int64)
    slot_tok = np.repeat(toks, k)
    slot_ex = np.maximum(idx[toks].reshape(-1), 0)   # unused slots (-1) are never kept
    kept_mask = dsp["row_of"][toks].reshape(-1) >= 0
    d = xr.shape[1]
    d_ff = _raw(w_gate)[0].shape[2]
    o_slots = np.zeros((toks.shape[0] * k, d), dtype=np.float64)
    h_slots = np.zeros((toks.shape[0] * k, d_ff), dtype=np.float64) if want_h else None
    sel = np.nonzero(kept_mask)[0]
    res = ffn_rows(slot_tok[sel], slot_ex[sel], x, w_gate, w_up, w_down, want_h=want_h)
    if want_h:
        h_slots[sel], o_slots[sel] = res
    else:
        o_slots[sel] = res
    y = combine(toks, dsp["row_of"], gate, o_slots)
    out = dict(logits=lg, idx=idx, gate=gate, C=C, tokens=toks, o_slots=o_slots, y=y)
    out.update(dsp)
    if want_h:
        out["h_slots"] = h_slots
    return out

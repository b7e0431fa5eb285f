"""The layer's expert FFN, combine and backward in fp64, one expert's rows at a
time, with numpy's fp64 matrix product as the step for every sum over the
model or FFN width.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this module.  It never imports the
HIP library or its binding.

Why it exists: the row-by-row C oracle (moe_oracle.c) streams every weight of
an expert once per row and needs minutes for the large layers; here each
expert's rows are gathered into a block and multiplied by that expert's
weights with a library matrix product, so every output of a full-size layer
can be checked against fp64 values.  Nothing else changes: the same
definitions, the same steps in the same order, no intermediate rounding
(all values are exact fp64 widenings of the inputs).  Its results agree with
the C oracle's to fp64 rounding (tests/test_oracle_by_expert.py pins that,
and the C oracle itself is pinned to library routines, brute force, closed
forms and finite differences).

Definitions (pages cited by title and section):
  * expert FFN, GeGLU ("AMD GPU深度学习优化与ZAYA1大模型实践", section 3.2, GeGLU
    fused with the matmul; expert-FFN shape: "AMD MI300X平台上的MoE模型训练实践",
    section 2.1): for a row of token t routed to expert e,
      g = x_t Wg[e],  u = x_t Wu[e],  h = GELU(g) * u,  o = h Wd[e],
    GELU in its erf form, GELU(v) = v (1 + erf(v / sqrt 2)) / 2.
  * combine: y_t = sum over the kept choices j of gate_tj * o_(t, j); a token
    with nothing kept gets y_t = 0 (the terms of one token arrive expert by
    expert here; with fp64 the order of a sum of k <= 8 terms is immaterial
    at the tolerances the tests use).
  * backward (the layer is trained on every page, e.g. the TorchTitan 1K-GPU
    article, section 2): the derivative of the forward above for an upstream
    gradient dy, with routing and drops held fixed (they are piecewise
    constant): per kept row of expert e with gate a,
      dgate = dy_t . o,  dO = a dy_t,  dh = dO Wd[e]^T,
      du = dh GELU(g),   dg = dh u GELU'(g),
      dWd[e] += h^T dO,  dWg[e] += x_t^T dg,  dWu[e] += x_t^T du,
      dx_t += dg Wg[e]^T + du Wu[e]^T,
    then the router: dlogit from dgate through the renormalised (or raw)
    gates and the temperature softmax (C oracle, orc_router_backward),
    dWr = x^T dlogit, db = sum_t dlogit, dx_t += dlogit_t Wr^T.
"""
from __future__ import annotations

from typing import Callable, Dict, Iterator, Optional, Tuple

import numpy as np
from scipy.special import erf

from . import oracle as orc

_SQRT2 = np.sqrt(2.0)
_SQRT2PI = np.sqrt(2.0 * np.pi)


def widen(a) -> np.ndarray:
    """Exact fp64 values of an fp32 or bf16 array (torch tensor or numpy)."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            return a.detach().cpu().double().numpy()
    except ImportError:  # pragma: no cover
        pass
    a = np.asarray(a)
    if a.dtype in (np.uint16, np.int16):   # raw bf16 patterns
        return (a.view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def gelu(v: np.ndarray) -> np.ndarray:
    """GELU in its erf form, v * Phi(v)."""
    return 0.5 * v * (1.0 + erf(v / _SQRT2))


def gelu_grad(v: np.ndarray) -> np.ndarray:
    """Derivative of the erf-form GELU: Phi(v) + v phi(v)."""
    return 0.5 * (1.0 + erf(v / _SQRT2)) + v * np.exp(-0.5 * v * v) / _SQRT2PI


def expert_ffn(x_rows: np.ndarray, wg: np.ndarray, wu: np.ndarray,
               wd: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """GeGLU FFN of one expert over a block of rows (fp64): returns (h, o)."""
    g = x_rows @ wg
    u = x_rows @ wu
    h = gelu(g) * u
    return h, h @ wd


def expert_blocks(offset, token_of_row, chunk: int = 8192) -> Iterator[Tuple[int, int, int]]:
    """(e, r0, r1): expert e's rows r0 .. r1-1, in blocks of at most ``chunk``."""
    offset = np.asarray(offset)
    for e in range(len(offset) - 1):
        for r0 in range(int(offset[e]), int(offset[e + 1]), chunk):
            yield e, r0, min(r0 + chunk, int(offset[e + 1]))


def forward_rows(x, w_gate, w_up, w_down, offset, token_of_row,
                 chunk: int = 8192) -> Iterator[Tuple[int, int, int, np.ndarray, np.ndarray]]:
    """Expert FFN of every kept row, block by block: yields (e, r0, r1, h, o)
    for rows r0 .. r1-1 of expert e (row r holds token token_of_row[r]).
    x [T, d], w_gate / w_up [E, d, d_ff], w_down [E, d_ff, d]; fp32 or bf16
    (torch CPU tensors or numpy), widened exactly to fp64."""
    token_of_row = np.asarray(token_of_row)
    cur, W = -1, None
    for e, r0, r1 in expert_blocks(offset, token_of_row, chunk):
        if e != cur:
            W = (widen(w_gate[e]), widen(w_up[e]), widen(w_down[e]))
            cur = e
        xr = widen(x[token_of_row[r0:r1]])
        h, o = expert_ffn(xr, *W)
        yield e, r0, r1, h, o


def row_gates(row_of: np.ndarray, gate: np.ndarray, n_rows: int) -> np.ndarray:
    """gate of the assignment each row holds (rows hold kept assignments)."""
    row_of = np.asarray(row_of)
    g = np.zeros(n_rows, dtype=np.float64)
    kept = row_of >= 0
    g[row_of[kept]] = np.asarray(gate, dtype=np.float64)[kept]
    return g


def combine_add(y: np.ndarray, tokens: np.ndarray, gates: np.ndarray, o: np.ndarray) -> None:
    """y[t] += gate * o for a block of rows of one expert (its tokens are
    distinct: a token chooses an expert at most once)."""
    y[tokens] += gates[:, None] * o


def forward_full(x, w_gate, w_up, w_down, offset, token_of_row, row_of, gate, T: int,
                 chunk: int = 8192,
                 on_block: Optional[Callable[[int, int, int, np.ndarray, np.ndarray], None]] = None
                 ) -> np.ndarray:
    """y [T, d] of the whole layer for the given routing (every row, every
    token), calling on_block(e, r0, r1, h, o) for each block of rows."""
    token_of_row = np.asarray(token_of_row)
    d = x.shape[1]
    n = int(np.asarray(offset)[-1])
    rg = row_gates(row_of, gate, n)
    y = np.zeros((T, d), dtype=np.float64)
    for e, r0, r1, h, o in forward_rows(x, w_gate, w_up, w_down, offset, token_of_row, chunk):
        if on_block is not None:
            on_block(e, r0, r1, h, o)
        combine_add(y, token_of_row[r0:r1], rg[r0:r1], o)
    return y


def backward(x, w_router, w_gate, w_up, w_down, dy, *, logits, idx, gate, row_of, offset,
             token_of_row, tau: float, renormalize: bool, chunk: int = 8192,
             on_expert: Optional[Callable[[int, Dict[str, np.ndarray]], None]] = None
             ) -> Dict[str, np.ndarray]:
    """Every gradient of the layer (fp64) for an upstream gradient dy [T, d]
    and the given routing (logits [T, E] the values it ranked, idx / gate /
    row_of [T, k], offset [E + 1], token_of_row).  Expert weight gradients go
    to on_expert(e, {"dw_gate", "dw_up", "dw_down"}) when given (so a caller
    can compare them expert by expert), else into the returned dict."""
    token_of_row = np.asarray(token_of_row)
    row_of = np.asarray(row_of)
    T, d = x.shape
    E = w_router.shape[1]
    k = row_of.shape[1]
    d_ff = w_gate.shape[2]
    n = int(np.asarray(offset)[-1])
    rg = row_gates(row_of, gate, n)
    # row -> flat (t, j) slot
    slot = np.full(n, -1, dtype=np.int64)
    kept = row_of >= 0
    slot[row_of[kept]] = np.nonzero(kept.ravel())[0]
    dy64 = widen(dy)
    dx = np.zeros((T, d), dtype=np.float64)
    dgate = np.zeros((T, k), dtype=np.float64)
    store = on_expert is None
    if store:
        out_w = {nm: np.zeros((E,) + sh) for nm, sh in
                 (("dw_gate", (d, d_ff)), ("dw_up", (d, d_ff)), ("dw_down", (d_ff, d)))}
    off = np.asarray(offset)
    for e in range(E):
        wg, wu, wd = widen(w_gate[e]), widen(w_up[e]), widen(w_down[e])
        dwg = np.zeros((d, d_ff))
        dwu = np.zeros((d, d_ff))
        dwd = np.zeros((d_ff, d))
        for r0 in range(int(off[e]), int(off[e + 1]), chunk):
            r1 = min(r0 + chunk, int(off[e + 1]))
            toks = token_of_row[r0:r1]
            xr = widen(x[toks])
            g = xr @ wg
            u = xr @ wu
            act = gelu(g)
            h = act * u
            o = h @ wd
            dyr = dy64[toks]
            dgate.ravel()[slot[r0:r1]] = np.einsum("rc,rc->r", dyr, o)
            dO = rg[r0:r1, None] * dyr
            dh = dO @ wd.T
            du = dh * act
            dg = dh * u * gelu_grad(g)
            dwd += h.T @ dO
            dwg += xr.T @ dg
            dwu += xr.T @ du
            dx[toks] += dg @ wg.T + du @ wu.T
        grads = {"dw_gate": dwg, "dw_up": dwu, "dw_down": dwd}
        if store:
            for nm, v in grads.items():
                out_w[nm][e] = v
        else:
            on_expert(e, grads)
    dl = orc.router_backward(logits, idx, gate, dgate, tau, renormalize)
    x64 = widen(x)
    wr64 = widen(w_router)
    dx += dl @ wr64.T
    out = {"dx": dx, "dgate": dgate, "dlogits": dl, "dw_router": x64.T @ dl,
           "dbias": dl.sum(axis=0)}
    if store:
        out.update(out_w)
    return out

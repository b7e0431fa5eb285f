"""Shared helpers of the GPU parity tests: input placement, tolerance
formulas and the oracle comparisons.  The expected values always come from
the fp64 oracle; nothing here computes a step of the layer itself."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import mixture_experts_layer_15_amd as moe
from mixture_experts_layer_15_amd import synthetic
from oracle import by_expert
from oracle import oracle as orc

U32 = 2.0 ** -24          # unit roundoff of fp32
TOL_Y = {"bf16": 2e-2, "f32": 1e-5}   # max |y - y*| / max |y*| over the output


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def gpu_inputs(cfg, seed=0):
    """Inputs on the GPU plus host copies for the oracle.  Small layers are
    drawn on the CPU (identical everywhere); large ones on the GPU."""
    small = cfg.E * cfg.d * cfg.d_ff <= (1 << 24) and cfg.T * cfg.d <= (1 << 24)
    if small:
        host = synthetic.make_inputs(cfg, seed=seed, device="cpu")
        dev = {k: (None if v is None else v.cuda()) for k, v in host.items()}
    else:
        dev = synthetic.make_inputs(cfg, seed=seed, device="cuda")
        torch.cuda.synchronize()
        host = {k: (None if v is None else v.cpu()) for k, v in dev.items()}
    return dev, host


def rel_err(got, want) -> float:
    """max |got - want| / max |want| (0 when both are exactly zero)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    scale = np.abs(want).max() if want.size else 0.0
    diff = np.abs(got - want).max() if want.size else 0.0
    if scale == 0.0:
        return 0.0 if diff == 0.0 else math.inf
    return diff / scale


def check_logits(logits_gpu, x_host, wr_host, bias_host, tokens, chunk=8192):
    """GPU fp32 logits against the oracle's fp64 logits within the fp32
    summation bound |l - l*| <= 2 g_K sum_i |x_i w_i| + 2u |l*| (+ bias term),
    g_K = K u / (1 - K u) (the factor 2 covers the MFMA's internal order).
    Returns the oracle's fp64 logits of the listed tokens."""
    tokens = np.asarray(tokens)
    K = x_host.shape[1]
    gk = K * U32 / (1 - K * U32)
    aw = np.abs(wr_host.double().numpy())
    wants = []
    for c0 in range(0, tokens.size, chunk):
        tk = tokens[c0:c0 + chunk]
        xs = x_host[torch.from_numpy(tk)]
        want = orc.logits(xs, wr_host, bias_host)
        ax = np.abs(xs.double().numpy())
        bound = 2 * gk * (ax @ aw) + 2 * U32 * np.abs(want) + 1e-30
        got = logits_gpu[torch.from_numpy(tk)].double().numpy()
        over = np.abs(got - want) > bound
        assert not over.any(), f"logits outside the fp32 bound at tokens {tk[np.argwhere(over)[:5, 0]]}"
        wants.append(want)
    return np.concatenate(wants) if wants else np.zeros((0, wr_host.shape[1]))


def dynamic_margin(cfg, lg):
    """For a layer with a dynamic expert count: per token, the smallest
    |cumulative softmax mass - threshold| over the decisions the count makes
    (fp64).  Both sides decide in fp64 with different summation orders, so a
    token whose margin is below 1e-12 may legitimately differ."""
    tau = float(np.float32(cfg.temperature))
    z = (lg - lg.max(1, keepdims=True)) / tau
    p = np.exp(z)
    p /= p.sum(1, keepdims=True)
    order = np.lexsort((np.broadcast_to(np.arange(lg.shape[1]), lg.shape), -lg), axis=1)
    cs = np.cumsum(np.take_along_axis(p, order, 1)[:, :cfg.k], 1)
    th = float(np.float32(cfg.route_threshold))
    return np.abs(cs[:, cfg.k_min - 1:] - th).min(1)


def check_route(cfg, logits_gpu, idx_gpu, gate_gpu):
    """Same-fp32-logits protocol: the oracle routes the GPU's logits; indices
    must match exactly, gates within an fp32 error bound of the softmax.  With
    a dynamic expert count, the (fp64) count decisions must match too, except
    for tokens whose cumulative mass lies within 1e-12 of the threshold."""
    lg = logits_gpu.double().numpy()
    tau = float(np.float32(cfg.temperature))
    dyn = getattr(cfg, "route_threshold", 0.0) > 0
    oidx, ogate = orc.route(lg, cfg.k, tau, cfg.renormalize,
                            cfg.k_min if dyn else 0,
                            float(np.float32(cfg.route_threshold)) if dyn else 0.0)
    gidx = idx_gpu.numpy()
    if dyn and lg.shape[0]:
        near = dynamic_margin(cfg, lg) < 1e-12
        say(f"dynamic expert count: {int(near.sum())} tokens within 1e-12 of the threshold; "
            f"tokens taking 1..{cfg.k} experts: "
            f"{np.bincount((oidx >= 0).sum(1), minlength=cfg.k + 1)[1:].tolist()}")
        gidx = np.where(near[:, None], oidx, gidx)
    bad = np.argwhere(gidx != oidx)
    assert bad.size == 0, f"top-k differs at {bad[:5]}: gpu {gidx[bad[0][0]]} oracle {oidx[bad[0][0]]}"
    # fp32 gate error: exp argument (l_j - max)/tau rounded twice and amplified by
    # exp, plus the sum of E terms and the division
    a = (np.take_along_axis(lg, np.maximum(oidx, 0), 1) - lg.max(1, keepdims=True)) / tau
    # below fp32's normal range (2^-126) there is no relative precision left (and
    # the hardware may flush to zero): an absolute slack of 2^-126 covers that
    tol = (4 * np.abs(a) + 2 * cfg.E + 24) * U32 * ogate + 2.0 ** -126
    g = gate_gpu.double().numpy()
    err = np.abs(g - ogate)
    bad = err > tol
    assert not bad.any(), f"gate error {err[bad].max():.3g} above bound at {np.argwhere(bad)[:5]}"
    used = ogate > 0          # slots past a token's dynamic count hold gate 0 on both sides
    rel = err[used] / ogate[used]
    return oidx, ogate, float(rel.max()) if rel.size else 0.0


def oracle_capacity(cfg, oidx):
    """The capacity the oracle applies: from the realised assignments with a
    dynamic expert count, else from T * k."""
    if getattr(cfg, "route_threshold", 0.0) > 0:
        return orc.capacity_realised(oidx, cfg.E, cfg.cap_num, cfg.cap_den)
    return orc.capacity(cfg.T, cfg.E, cfg.k, cfg.cap_num, cfg.cap_den)


def check_dispatch(cfg, oidx, dsp):
    """Integer outputs of dispatch bit-exact against the oracle."""
    C = oracle_capacity(cfg, oidx)
    od = orc.dispatch(oidx, cfg.E, C, cfg.drop_policy)
    n = od["n_kept"]
    np.testing.assert_array_equal(dsp["expert_count"].cpu().numpy(), od["count"])
    np.testing.assert_array_equal(dsp["expert_offset"].cpu().numpy(), od["offset"])
    np.testing.assert_array_equal(dsp["row_of"].cpu().numpy(), od["row_of"])
    tor = dsp["token_of_row"].cpu().numpy()
    np.testing.assert_array_equal(tor[:n], od["token_of_row"])
    assert (tor[n:] == -1).all()
    return od


def check_x_perm(x_dev, x_perm, token_of_row, n):
    """x_perm[r] is byte-for-byte x[token_of_row[r]] for every kept row."""
    if n == 0:
        return
    tor = torch.from_numpy(np.ascontiguousarray(token_of_row[:n])).long().cuda()
    a = x_perm[:n]
    b = x_dev.index_select(0, tor)
    iv = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
    assert torch.equal(a.view(iv), b.view(iv)), "x_perm rows differ from x"


def expert_of_rows(offset, rows):
    return np.searchsorted(offset, rows, side="right") - 1


def sample_rows(offset, n, full, rng, extra=96):
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    if full:
        return np.arange(n)
    pick = set()
    E = len(offset) - 1
    for e in range(E):
        if offset[e + 1] > offset[e]:
            pick.update({int(offset[e]), int(offset[e + 1] - 1)})
    pick.update(rng.integers(0, n, size=extra).tolist())
    return np.array(sorted(pick), dtype=np.int64)


def to_np(t):
    return t.float().cpu().double().numpy() if t.dtype == torch.bfloat16 else t.cpu().double().numpy()


def fused_down_split(cfg) -> bool:
    """Whether moe_forward runs this layer's down GEMM in two K slices (fp32
    partials summed by a second kernel): bf16, top-1, compact layout, every
    token kept, at most 2048 rows per expert on average, and too few
    320 x 256 down tiles (E * ceil(d / 256)) to fill the CUs.  Its output then
    differs from the staged calls' by the fp32 summation order only."""
    import torch
    if cfg.dtype != "bf16" or cfg.k != 1 or cfg.layout != 0 or cfg.T == 0:
        return False
    cap = cfg.T if cfg.cap_den == 0 else -(-cfg.cap_num * cfg.k * cfg.T // (cfg.cap_den * cfg.E))
    if cap < cfg.T:
        return False
    rows = cfg.T * cfg.k
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return (rows <= 2048 * cfg.E and cfg.E * -(-cfg.d // 256) < cus and cfg.d_ff % 128 == 0)


def bf16_ulp_distance(a, b) -> int:
    """Largest distance, in units in the last place, between two bf16 tensors
    of the same shape (+0 and -0 are the same value)."""
    import torch
    def key(t):
        u = t.contiguous().view(torch.int16).to(torch.int32) & 0xFFFF
        mag = u & 0x7FFF
        return torch.where((u & 0x8000) != 0, -mag, mag)
    if a.numel() == 0:
        return 0
    return int((key(a) - key(b)).abs().max().item())



class MaxRel:
    """Running max |got - want| and max |want| over blocks of one output, for
    the R13 measure max |got - want| / max |want| over the whole output."""

    def __init__(self):
        self.diff = 0.0
        self.scale = 0.0
        self.count = 0

    def add(self, got, want):
        got = np.asarray(got, dtype=np.float64)
        want = np.asarray(want, dtype=np.float64)
        if want.size:
            assert np.isfinite(got).all(), "non-finite values (an unwritten element?)"
            self.diff = max(self.diff, float(np.abs(got - want).max()))
            self.scale = max(self.scale, float(np.abs(want).max()))
            self.count += want.shape[0]

    def value(self) -> float:
        if self.scale == 0.0:
            return 0.0 if self.diff == 0.0 else math.inf
        return self.diff / self.scale


def check_ffn_and_combine_by_expert(cfg, host, od, ogate, h, y_perm, label, chunk=8192):
    """Every row of h and y_perm, and the fp64 layer output y* of every token,
    from the by-expert oracle (fp64 matrix products per expert block) on the
    oracle's routing (ogate: its fp64 gates) and dispatch od.  Returns y*."""
    mh, mo = MaxRel(), MaxRel()
    n = od["n_kept"]

    def on_block(e, r0, r1, hb, ob):
        mh.add(to_np(h[r0:r1]), hb)
        mo.add(to_np(y_perm[r0:r1]), ob)

    ystar = by_expert.forward_full(host["x"], host["w_gate"], host["w_up"], host["w_down"],
                                   od["offset"], od["token_of_row"], od["row_of"], ogate,
                                   cfg.T, chunk=chunk, on_block=on_block)
    assert mh.count == n and mo.count == n
    eh, eo = mh.value(), mo.value()
    say(f"[{label}] h err {eh:.3g}  y_perm err {eo:.3g} over all {n} rows")
    assert eh <= TOL_Y[cfg.dtype] and eo <= TOL_Y[cfg.dtype]
    return ystar

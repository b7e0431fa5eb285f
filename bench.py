"""Benchmark of the MoE FFN forward on one MI355X.

A step is one pass of the whole layer -- route, dispatch, gate/up GEMM, down
GEMM, combine -- over one batch of synthetic tokens, through the C ABI.
Inputs sit in HBM before the timed region; the token batch rotates over
several copies so that no step finds its activations in the 256 MB
last-level cache (the weights, 1.6 GB here, never fit).  Two timed regions:
the fused entry point moe_forward gives the step time and `value` (tokens/s);
the same steps through the five per-stage entry points, with HIP events
recorded on the launch stream between them, give each stage's time (and the
roofline of the dominant kernel).

Prints ONE JSON line.  Default workload: the ZAYA1-like layer (T = 4096,
d = 2048, E = 16, top-1, GeGLU d_ff = 8192, bf16).  ``--config`` selects
another of the five layers for manual runs.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3       # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
METRIC = "MoE fwd tokens/s + grouped-GEMM TFLOP/s (% bf16 MFMA peak) on 1 MI355X"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="zaya1")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the moe_backward timing (e.g. for counter runs of the forward)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MB",
                    help="only run a plain device copy of MB megabytes (5 times) and exit: the "
                         "known-size reference for scaling FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


def algorithmic(cfg, counts, n_kept):
    """Bytes and flops each stage must move / do (padding and dropped rows excluded)."""
    b = 2 if cfg.dtype == "bf16" else 4
    T, d, E, k, F = cfg.T, cfg.d, cfg.E, cfg.k, cfg.d_ff
    ne = sum(1 for c in counts if c > 0)
    return {
        "route_bytes": T * d * b + d * E * b + T * E * 4 + T * k * 8,
        "dispatch_bytes": None,   # filled by caller (needs active-token count)
        "gate_up_flops": 4.0 * d * F * n_kept,
        "gate_up_bytes": 2 * ne * d * F * b + n_kept * d * b + n_kept * F * b,
        "down_flops": 2.0 * d * F * n_kept,
        "down_bytes": ne * F * d * b + n_kept * F * b + n_kept * d * b,
        "combine_bytes": n_kept * d * b + T * d * b + T * k * 8,
    }


def roofline(cfg, a, launch_ms, peak, traffic, traffic_kernel):
    """Roofline of the dominant kernel (gate/up GEMM + GeGLU): bound by whichever
    of HBM bytes or matrix/vector flops takes longer at the chip's peak; achieved
    = that algorithmic quantity / the average launch time."""
    t_hbm = a["gate_up_bytes"] / (PEAK_HBM_GBS * 1e9)
    t_alu = a["gate_up_flops"] / (peak * 1e12)
    sec = launch_ms * 1e-3
    r = {"kernel": traffic_kernel or ("gemm_mfma_kernel<true, ...> (gate/up + GeGLU)"
                                       if cfg.dtype == "bf16" else
                                       "grouped_gemm_f32_kernel<true> (gate/up + GeGLU)")}
    if t_hbm >= t_alu:
        ach = a["gate_up_bytes"] / sec / 1e9
        r.update(bound="hbm", achieved=round(ach, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                 frac=round(ach / PEAK_HBM_GBS, 4))
    else:
        ach = a["gate_up_flops"] / sec / 1e12
        r.update(bound="mfma" if cfg.dtype == "bf16" else "alu", achieved=round(ach, 1),
                 peak=peak, unit="TFLOP/s", frac=round(ach / peak, 4))
    r.update(traffic=traffic, traffic_unit="bytes per launch",
             algorithmic_bytes_per_launch=a["gate_up_bytes"],
             flops_per_launch=a["gate_up_flops"],
             hbm_frac=round(a["gate_up_bytes"] / sec / 1e9 / PEAK_HBM_GBS, 4),
             flops_frac=round(a["gate_up_flops"] / sec / 1e12 / peak, 4),
             avg_launch_ms=round(launch_ms, 4))
    return r


def mlp_router_ms(cfg, xs, n_rot, K):
    """Mean time of moe_route_mlp (the ZAYA1 MLP router variant, r = 256,
    m = 1024, seeded random weights) over K calls, HIP events on the stream."""
    import torch
    import mixture_experts_layer_15_amd as moe
    g = torch.Generator(device="cuda").manual_seed(1)
    n = lambda *sh, sc=1.0: torch.randn(*sh, generator=g, device="cuda") * sc
    r, m = 256, 1024
    rt = dict(w_down=n(cfg.d, r, sc=cfg.d ** -0.5).bfloat16(), b_down=n(r, sc=0.1),
              w1=n(r, m, sc=r ** -0.5).bfloat16(), b1=n(m, sc=0.1),
              w2=n(m, m, sc=m ** -0.5).bfloat16(), b2=n(m, sc=0.1),
              w3=n(m, cfg.E, sc=m ** -0.5).bfloat16(), b3=n(cfg.E, sc=0.1),
              pid_bias=n(cfg.E, sc=0.05))
    prev = n(cfg.T, r).bfloat16()
    for i in range(3):
        moe.route_mlp(cfg, xs[i % n_rot], prev, rt, 0.5, 1e-6)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(K):
        moe.route_mlp(cfg, xs[i % n_rot], prev, rt, 0.5, 1e-6)
    b.record()
    torch.cuda.synchronize()
    return round(a.elapsed_time(b) / K, 4)


def padded_forward_ms(cfg, dev, xs, n_rot, K):
    """Mean time of moe_forward with the padded-capacity layout (every expert
    runs C rows) over K calls, HIP events on the stream; None without a
    capacity limit."""
    import torch
    import mixture_experts_layer_15_amd as moe
    if cfg.cap_den == 0:
        return None
    pad = cfg.scaled(layout=moe.MOE_LAYOUT_PADDED)
    fwd = moe.Forward(pad)
    args = (dev["w_router"], dev["bias"], dev["w_gate"], dev["w_up"], dev["w_down"])
    y = fwd(xs[0], *args)
    for i in range(1, 3):
        fwd(xs[i % n_rot], *args, y=y)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(K):
        fwd(xs[i % n_rot], *args, y=y)
    b.record()
    torch.cuda.synchronize()
    return round(a.elapsed_time(b) / K, 4)


def backward_ms(cfg, dev, xs, n_rot, K):
    """Mean time of moe_backward (recompute of routing and pre-activations,
    every gradient) over K calls with preallocated outputs and workspace,
    HIP events on the stream; dy ~ N(0, 1)."""
    import torch
    import mixture_experts_layer_15_amd as moe
    from mixture_experts_layer_15_amd import synthetic
    dy = synthetic.make_dy(cfg, seed=1, device="cuda")
    bw = moe.Backward(cfg)
    args = (dev["w_router"], dev["bias"], dev["w_gate"], dev["w_up"], dev["w_down"], dy)
    out = bw(xs[0], *args)
    for i in range(1, 3):
        bw(xs[i % n_rot], *args, out=out)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(K):
        bw(xs[i % n_rot], *args, out=out)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / K


GEMM_SOURCES = ("gemm_mfma.hip", "tiles.h", "lds_dma.h", "common.h")


def gemm_source_hash() -> str:
    """First 16 hex digits of the SHA-256 over the gate/up kernel's sources (the
    kernel file and the headers it includes, in this order)."""
    import hashlib
    h = hashlib.sha256()
    for name in GEMM_SOURCES:
        h.update(open(os.path.join(ROOT, "mixture_experts_layer_15_amd", "csrc", name), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(cfg):
    """HBM bytes per launch of the gate/up GEMM from the committed FETCH_SIZE /
    WRITE_SIZE counter runs (scaled by a plain copy of known size), or None when
    they were taken on another workload or the GEMM sources have changed since."""
    path = os.path.join(ROOT, "profiles", f"traffic_gemm_gate_up_{cfg.name}.json")
    if not os.path.exists(path):
        return None, None
    rec = json.load(open(path))
    if rec.get("gemm_source_sha256_16") != gemm_source_hash():
        return None, None
    return rec["traffic_bytes_per_launch"], rec["kernel"]


def cpu_baseline(cfg, host, logits_gpu, target_s):
    """The fp64 oracle, as it stands, on a bounded sample of the same batch:
    routing + capacity + dispatch of every token, then the GeGLU FFN and
    combine of a token sample sized to about target_s seconds; scaled to the
    whole batch."""
    import numpy as np
    from oracle import oracle as orc
    kw = dict(k=cfg.k, tau=float(np.float32(cfg.temperature)), renormalize=cfg.renormalize,
              cap_num=cfg.cap_num, cap_den=cfg.cap_den)
    t0 = time.perf_counter()
    lg = orc.logits(host["x"], host["w_router"], host["bias"])
    idx, gate = orc.route(lg, cfg.k, kw["tau"], cfg.renormalize)
    C = orc.capacity(cfg.T, cfg.E, cfg.k, cfg.cap_num, cfg.cap_den)
    orc.dispatch(idx, cfg.E, C)
    t_route = time.perf_counter() - t0
    # probe the per-token FFN cost, then size the sample
    probe = 16
    t0 = time.perf_counter()
    orc.forward(host["x"], host["w_router"], host["bias"], host["w_gate"], host["w_up"],
                host["w_down"], logits_in=lg, tokens=list(range(probe)), **kw)
    t_probe = time.perf_counter() - t0
    per_tok = max(t_probe / probe, 1e-6)
    n = int(min(cfg.T, max(probe, target_s / per_tok)))
    rng = np.random.default_rng(1)
    toks = np.sort(rng.choice(cfg.T, size=n, replace=False))
    t0 = time.perf_counter()
    orc.forward(host["x"], host["w_router"], host["bias"], host["w_gate"], host["w_up"],
                host["w_down"], logits_in=lg, tokens=toks, **kw)
    t_ffn = time.perf_counter() - t0
    total = t_route + t_ffn * cfg.T / n
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": cfg.T / total, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": (f"fp64 oracle: logits, top-k, capacity and dispatch of all {cfg.T} tokens "
                       f"({t_route:.2f} s) + GeGLU FFN and combine of {n} random tokens "
                       f"({t_ffn:.2f} s), scaled to {cfg.T} tokens"),
            "seconds_measured": round(t_route + t_ffn, 2)}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "this layer's forward is measured on a single MI355X.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mixture_experts_layer_15_amd as moe
    from mixture_experts_layer_15_amd import configs, synthetic

    if args.copy_calibration:
        n = args.copy_calibration * 2 ** 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 5}), flush=True)
        return

    cfg = configs.get(args.config)
    torch.cuda.set_device(0)
    dev = synthetic.make_inputs(cfg, seed=0, device="cuda")
    x0 = dev["x"]
    xb = x0.numel() * x0.element_size()
    n_rot = max(1, min(64, -(-512 * 2 ** 20 // xb)))   # >= 512 MB of distinct token batches
    xs = [x0] + [x0.roll(i, dims=0).contiguous() for i in range(1, n_rot)]
    wr, bias, wg, wu, wd = dev["w_router"], dev["bias"], dev["w_gate"], dev["w_up"], dev["w_down"]

    R = moe.max_rows(cfg)
    dt = x0.dtype
    logits = torch.empty((cfg.T, cfg.E), dtype=torch.float32, device="cuda")
    idx = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
    gate = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device="cuda")
    x_perm = torch.empty((R, cfg.d), dtype=dt, device="cuda")
    count = torch.empty(cfg.E, dtype=torch.int32, device="cuda")
    offset = torch.empty(cfg.E + 1, dtype=torch.int32, device="cuda")
    row_of = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
    tor = torch.empty(cfg.T * cfg.k, dtype=torch.int32, device="cuda")
    h = torch.empty((R, cfg.d_ff), dtype=dt, device="cuda")
    y_perm = torch.empty((R, cfg.d), dtype=dt, device="cuda")
    y = torch.empty((cfg.T, cfg.d), dtype=dt, device="cuda")
    dws = moe.workspace_bytes(cfg, dispatch_only=True)
    dsp_ws = torch.empty(max(dws, 16), dtype=torch.uint8, device="cuda")

    L = moe.lib()
    c = moe.cconfig(cfg)
    P = moe._ptr
    import ctypes
    cref = ctypes.byref(c)

    def step(x, ev=None):
        s = moe._stream()
        if ev: ev[0].record()
        moe._check(L.moe_route(cref, P(x), P(wr), P(bias), P(logits), P(idx), P(gate), s), "route")
        if ev: ev[1].record()
        moe._check(L.moe_dispatch(cref, P(idx), P(x), P(x_perm), P(count), P(offset), P(row_of),
                                  P(tor), P(dsp_ws), dws, s), "dispatch")
        if ev: ev[2].record()
        moe._check(L.moe_expert_gate_up(cref, P(x_perm), P(offset), P(wg), P(wu), P(h), s), "gate_up")
        if ev: ev[3].record()
        moe._check(L.moe_expert_down(cref, P(h), P(offset), P(wd), P(y_perm), s), "down")
        if ev: ev[4].record()
        moe._check(L.moe_combine(cref, P(y_perm), P(row_of), P(gate), P(y), s), "combine")
        if ev: ev[5].record()

    for i in range(args.warmup):
        step(xs[i % n_rot])
    torch.cuda.synchronize()

    K = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(xs[i % n_rot], evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    names = ["route", "dispatch", "gate_up", "down", "combine"]
    stage_ms = {n: float(np.mean([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(K)]))
                for j, n in enumerate(names)}
    gpu_ms = float(np.mean([evs[i][0].elapsed_time(evs[i][5]) for i in range(K)]))
    ms_step = wall * 1e3 / K

    mlp_ms = mlp_router_ms(cfg, xs, n_rot, K) if cfg.dtype == "bf16" else None
    padded_ms = padded_forward_ms(cfg, dev, xs, n_rot, K)
    bwd_ms = backward_ms(cfg, dev, xs, n_rot, K) \
        if cfg.dtype == "bf16" and not args.no_backward else None

    # the fused entry point: the step time that `value` reports
    fwd = moe.Forward(cfg)
    for i in range(3):
        fwd(xs[i % n_rot], wr, bias, wg, wu, wd, y)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(K):
        fwd(xs[i % n_rot], wr, bias, wg, wu, wd, y)
    torch.cuda.synchronize()
    fused_ms = (time.perf_counter() - t1) * 1e3 / K

    # algorithmic work of the last step's routing (same for every rotated batch
    # up to token order; recompute from the first batch for exactness)
    step(xs[0])
    torch.cuda.synchronize()
    ls = moe.load_stats(cfg, count).cpu().numpy()   # expert-load telemetry of this batch
    cnt = count.cpu().numpy()
    off = offset.cpu().numpy()
    n_kept = int(off[-1])
    rows = row_of.cpu().numpy()
    active = int((rows >= 0).any(1).sum())
    a = algorithmic(cfg, cnt, n_kept)
    b = 2 if cfg.dtype == "bf16" else 4
    a["dispatch_bytes"] = (active + n_kept) * cfg.d * b + cfg.T * cfg.k * 4 * 3 + \
        2 * 256 * cfg.E * 4
    gemm_ms = stage_ms["gate_up"] + stage_ms["down"]
    gemm_tflops = (a["gate_up_flops"] + a["down_flops"]) / (gemm_ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    gu_tflops = a["gate_up_flops"] / (stage_ms["gate_up"] * 1e-3) / 1e12

    def gbs(nbytes, ms):
        return nbytes / (ms * 1e-3) / 1e9

    traffic, traffic_kernel = measured_traffic(cfg)

    out = {
        "metric": METRIC,
        "value": round(cfg.T / (fused_ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(fused_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) tokens, N(0,1/fan_in) random-init weights)",
        "config": {"workload": f"{cfg.name}: T={cfg.T} d={cfg.d} E={cfg.E} top-{cfg.k} "
                               f"GeGLU d_ff={cfg.d_ff} {cfg.dtype}",
                   "T": cfg.T, "d": cfg.d, "E": cfg.E, "k": cfg.k, "d_ff": cfg.d_ff,
                   "temperature": cfg.temperature,
                   "capacity_factor": None if cfg.cap_den == 0 else cfg.cap_num / cfg.cap_den,
                   "rows_kept": n_kept, "parallelism": "single GPU"},
        "expert_load": {"mean": round(float(ls[0]), 2), "max": int(ls[1]), "min": int(ls[2]),
                        "max_over_mean": round(float(ls[3]), 4),
                        "max_deviation": round(float(ls[4]), 4), "cv": round(float(ls[5]), 4),
                        "dropped": int(ls[6]), "empty_experts": int(ls[7])},
        "variants": {"mlp_router_ms": mlp_ms,
                     "mlp_router_widths": "r=256 m=1024 (ZAYA1 MLP router, random weights)",
                     "padded_layout_ms_per_step": padded_ms},
        "backward": None if bwd_ms is None else {
            "ms_per_step": round(bwd_ms, 4),
            "tokens_per_s": round(cfg.T / (bwd_ms * 1e-3), 1),
            # recomputed g and u (2), dh (1), dx_perm (2), three weight gradients (3):
            # 8 products of 2 n_kept d d_ff flops each
            "gemm_tflops": round(16 * n_kept * cfg.d * cfg.d_ff / (bwd_ms * 1e-3) / 1e12, 1),
            "gemm_frac_of_peak": round(16 * n_kept * cfg.d * cfg.d_ff / (bwd_ms * 1e-3) / 1e12
                                       / peak, 4)},
        "grouped_gemm_tflops": round(gemm_tflops, 1),
        "grouped_gemm_frac_of_peak": round(gemm_tflops / peak, 4),
        "stage_ms": {k2: round(v, 4) for k2, v in stage_ms.items()},
        "stage_gbs": {"route": round(gbs(a["route_bytes"], stage_ms["route"]), 1),
                      "dispatch": round(gbs(a["dispatch_bytes"], stage_ms["dispatch"]), 1),
                      "combine": round(gbs(a["combine_bytes"], stage_ms["combine"]), 1)},
        "stage_hbm_frac": {"dispatch": round(gbs(a["dispatch_bytes"], stage_ms["dispatch"]) / PEAK_HBM_GBS, 4),
                           "combine": round(gbs(a["combine_bytes"], stage_ms["combine"]) / PEAK_HBM_GBS, 4)},
        "staged_ms_per_step": round(ms_step, 4),
        "staged_gpu_ms_per_step_events": round(gpu_ms, 4),
        "roofline": roofline(cfg, a, stage_ms["gate_up"], peak, traffic, traffic_kernel),
    }
    if not args.no_cpu_baseline:
        host = {k2: (None if v is None else v.cpu()) for k2, v in dev.items()}
        out["cpu_baseline"] = cpu_baseline(cfg, host, logits, args.cpu_seconds)
        out["cpu_baseline"]["value"] = round(out["cpu_baseline"]["value"], 2)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

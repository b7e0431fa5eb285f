"""Benchmark of the MoE FFN forward on one MI355X.

A step is one pass of the whole layer -- route, dispatch, gate/up GEMM, down
GEMM, combine -- over one batch of synthetic tokens, through the C ABI.
Inputs sit in HBM before the timed region; the token batch rotates over
several copies so that no step finds its activations in the 256 MB
last-level cache (the weights never fit).

Headline (`value`, `ms_per_step`): exactly --steps calls of the fused entry
point moe_forward on the long-sequence layer (T = 65,536 tokens x d = 6,144,
8 experts, top-2, GeGLU d_ff = 4,096, bf16: the largest layer that one GPU
holds), wall clock between two synchronisations.  The same run measures the
ZAYA1-like, wide and skewed layers the same way under `per_config`.  For
each layer, the five per-stage entry points first run at least 30 times (and
for at least a quarter second, which also brings the clocks up from idle)
with HIP events recorded on the launch stream between the stages: the medians
give each stage's time, the means the roofline of the dominant kernel (the
gate/up GEMM with its GeGLU epilogue).  Peak probes (a streaming copy and
read, a dense bf16 MFMA stream with clock stamps, and the vendor library's
bf16 GEMM on two expert shapes as a reference) run outside every timed
region, and the core clock is sampled from sysfs while the headline's
timed loop runs.  The fp64 oracle is timed on the host's cores on a bounded
token sample of each layer (`cpu_baseline`), and ranks its own fp64 logits
to count the tokens whose routing differs from the GPU's fp32 logits.  Each
layer also times moe_backward (`backward`) and, outside the timed regions, its
variants (`variants`: the padded-capacity layout and the choice-order drop
priority where a capacity limit applies, the MLP router at r = 256, m = 1024,
one PID controller step).

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import glob
import json
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3       # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
METRIC = "MoE fwd tokens/s + grouped-GEMM TFLOP/s (% bf16 MFMA peak) on 1 MI355X"
HEADLINE = "longseq"
OTHERS = ("zaya1", "wide", "skewed")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default=HEADLINE, help="the headline layer")
    ap.add_argument("--only-headline", action="store_true",
                    help="measure the headline layer only (e.g. for profiler runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the moe_backward timing (e.g. for counter runs of the forward)")
    ap.add_argument("--no-probes", action="store_true", help="skip the peak probes")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the timing of the layout, drop-priority and router variants")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the headline layer's oracle sample")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MB",
                    help="only run a plain device copy of MB megabytes (5 times) and exit: the "
                         "known-size reference for scaling FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


def median(v):
    s = sorted(v)
    n = len(s)
    return s[n // 2] if n % 2 else 0.5 * (s[n // 2 - 1] + s[n // 2])


def algorithmic(cfg, counts, n_kept, active):
    """Bytes and flops each stage must move / do (padding and dropped rows excluded)."""
    b = 2 if cfg.dtype == "bf16" else 4
    T, d, E, k, F = cfg.T, cfg.d, cfg.E, cfg.k, cfg.d_ff
    ne = sum(1 for c in counts if c > 0)
    return {
        "route_bytes": T * d * b + d * E * b + T * E * 4 + T * k * 8,
        # x rows read once per active token and written once per kept row,
        # plus the index arrays (idx read; row_of, token_of_row written) and
        # the two per-block count tables
        "dispatch_bytes": (active + n_kept) * d * b + T * k * 4 * 3 + 2 * 256 * E * 4,
        "gate_up_flops": 4.0 * d * F * n_kept,
        "gate_up_bytes": 2 * ne * d * F * b + n_kept * d * b + n_kept * F * b,
        "down_flops": 2.0 * d * F * n_kept,
        "down_bytes": ne * F * d * b + n_kept * F * b + n_kept * d * b,
        "combine_bytes": n_kept * d * b + T * d * b + T * k * 8,
    }


def roofline(cfg, a, launch_ms, peak, traffic, traffic_kernel, measured_peak=None):
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
    if measured_peak:
        r["frac_of_measured_peak"] = round(ach / measured_peak, 4)
    return r


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


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_threads() -> int:
    return int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))


class ClockSampler:
    """Samples the GPU core clock from sysfs (the level marked current in
    pp_dpm_sclk) every millisecond while a timed loop runs."""

    def __init__(self):
        paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.path = paths[0] if paths else None
        self.samples = []
        self._stop = threading.Event()
        self._t = None

    def _read(self):
        try:
            for line in open(self.path):
                if "*" in line:
                    return float(line.split(":", 1)[1].strip().rstrip("*").strip().lower()
                                 .replace("mhz", ""))
        except (OSError, ValueError, IndexError):
            return None
        return None

    def _run(self):
        while not self._stop.is_set():
            v = self._read()
            if v is not None:
                self.samples.append(v)
            time.sleep(0.001)

    def __enter__(self):
        if self.path:
            self._t = threading.Thread(target=self._run, daemon=True)
            self._t.start()
        return self

    def __exit__(self, *a):
        self._stop.set()
        if self._t:
            self._t.join()

    def summary(self):
        s = [v for v in self.samples if v > 0]
        if not s:
            return None
        busy = [v for v in s if v >= 1000]   # idle gaps between launches read as deep sleep
        use = busy or s
        return {"source": "sysfs pp_dpm_sclk (current level), sampled every 1 ms",
                "samples": len(s), "median_mhz": median(use), "min_mhz": min(use),
                "max_mhz": max(use)}


def run_probes(L, torch):
    """Streaming copy / read and dense bf16 MFMA throughput of this chip, with
    the core clock the MFMA stream ran at (outside every timed region)."""
    out = {"spec_peaks": {"hbm_gbs": PEAK_HBM_GBS, "mfma_bf16_tflops": PEAK_BF16_TFLOPS}}
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    nbytes = 2 << 30
    src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(8 * cus * 256, dtype=torch.float32, device="cuda")

    def timed(fn, reps=10):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        return ts

    L.moe_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                 ctypes.c_int32, ctypes.c_void_p]
    L.moe_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                 ctypes.c_int32, ctypes.c_void_p]
    L.moe_probe_mfma.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_void_p]
    for f in (L.moe_probe_copy, L.moe_probe_read, L.moe_probe_mfma):
        f.restype = ctypes.c_int

    def chk(st):
        if st != 0:
            raise RuntimeError(f"probe failed with status {st}")

    tc = timed(lambda: chk(L.moe_probe_copy(P(src), P(dst), nbytes, 0, s)))
    tr = timed(lambda: chk(L.moe_probe_read(P(src), nbytes, P(sink), 0, s)))
    out["hbm_copy_gbs"] = {"bytes_per_launch": 2 * nbytes,
                           "median": round(2 * nbytes / median(tc) / 1e9, 1),
                           "best": round(2 * nbytes / min(tc) / 1e9, 1)}
    out["hbm_read_gbs"] = {"bytes_per_launch": nbytes,
                           "median": round(nbytes / median(tr) / 1e9, 1),
                           "best": round(nbytes / min(tr) / 1e9, 1)}
    del src, dst
    blocks, iters = 2 * cus, 16384
    msink = torch.empty(blocks * 512, dtype=torch.float32, device="cuda")
    stamps = torch.zeros(blocks * 4, dtype=torch.int64, device="cuda")
    tm = timed(lambda: chk(L.moe_probe_mfma(blocks, iters, P(msink), P(stamps), s)))
    flops = blocks * 8 * iters * 8 * 16384
    st = stamps.view(blocks, 4).cpu().double()
    mhz = ((st[:, 1] - st[:, 0]) / ((st[:, 3] - st[:, 2]) / 100.0)).tolist()
    out["mfma_bf16_tflops"] = {"flops_per_launch": flops,
                               "median": round(flops / median(tm) / 1e12, 1),
                               "best": round(flops / min(tm) / 1e12, 1),
                               "core_clock_mhz_median": round(median(mhz), 1)}
    del msink, stamps
    # the vendor library's bf16 GEMM (torch.matmul -> hipBLASLt) on random
    # N(0, 1) data of two expert shapes: a reference for what a tuned library
    # reaches on this chip under its power limit, never part of the layer
    g = torch.Generator(device="cuda").manual_seed(0)
    ref = {}
    for name, (bt, M, K, N) in {"long_sequence_expert_gate_up": (1, 16384, 6144, 8192),
                                "zaya1_like_experts_gate_up": (16, 256, 2048, 16384)}.items():
        a = torch.randn(bt, M, K, generator=g, device="cuda", dtype=torch.bfloat16)
        b = (torch.randn(bt, K, N, generator=g, device="cuda") * K ** -0.5).to(torch.bfloat16)
        tv = timed(lambda: torch.bmm(a, b), reps=20)
        fl = 2.0 * bt * M * K * N
        ref[name] = {"shape": [bt, M, K, N], "median_ms": round(median(tv) * 1e3, 4),
                     "tflops": round(fl / median(tv) / 1e12, 1)}
        del a, b
    out["vendor_gemm_bf16"] = ref
    return out


def cpu_baseline(cfg, host, idx_gpu, row_of_gpu, target_s):
    """The fp64 oracle, as it stands, on a bounded sample of the same batch:
    logits, routing, capacity and dispatch of every token, then the GeGLU FFN
    and combine of a token sample sized to about target_s seconds; scaled to
    the whole batch.  Also ranks the oracle's own fp64 logits and counts the
    tokens whose routing differs from the GPU's (which ranks fp32 logits)."""
    import numpy as np
    from oracle import oracle as orc
    kw = dict(k=cfg.k, tau=float(np.float32(cfg.temperature)), renormalize=cfg.renormalize,
              cap_num=cfg.cap_num, cap_den=cfg.cap_den)
    dyn = dict(k_min=cfg.k_min, threshold=float(np.float32(cfg.route_threshold))) \
        if cfg.route_threshold > 0 else {}
    kw.update(dyn)
    t0 = time.perf_counter()
    lg = orc.logits(host["x"], host["w_router"], host["bias"])
    idx, gate = orc.route(lg, cfg.k, kw["tau"], cfg.renormalize, **dyn)
    C = orc.capacity_realised(idx, cfg.E, cfg.cap_num, cfg.cap_den) if dyn else \
        orc.capacity(cfg.T, cfg.E, cfg.k, cfg.cap_num, cfg.cap_den)
    od = orc.dispatch(idx, cfg.E, C)
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
    # fp64 flops the measured work did: router logits of every token, GeGLU FFN
    # (three d x d_ff products) of every kept assignment of the sampled tokens
    kept_sample = int((od["row_of"][toks] >= 0).sum())
    flops = 2.0 * cfg.T * cfg.d * cfg.E + 6.0 * cfg.d * cfg.d_ff * kept_sample
    topk_differs = ~(np.sort(idx, 1) == np.sort(idx_gpu, 1)).all(1)
    order_differs = ~(idx == idx_gpu).all(1)
    keep_differs = ((od["row_of"] >= 0) != (row_of_gpu >= 0)).any(1)
    base = {"value": round(cfg.T / total, 2), "unit": "tokens/s", "cores": oracle_threads(),
            "kind": "oracle",
            "sample": (f"fp64 oracle (C, OpenMP): logits, top-k, capacity and dispatch of all "
                       f"{cfg.T} tokens ({t_route:.2f} s) + GeGLU FFN and combine of {n} random "
                       f"tokens ({t_ffn:.2f} s), scaled to {cfg.T} tokens"),
            "seconds_measured": round(t_route + t_ffn, 2),
            "fp64_gflops": round(flops / (t_route + t_ffn) / 1e9, 1)}
    indep = {"tokens": cfg.T,
             "tokens_with_a_different_expert_set": int(topk_differs.sum()),
             "tokens_with_a_different_choice_order": int(order_differs.sum()),
             "tokens_with_a_different_keep_decision": int(keep_differs.sum()),
             "note": "oracle ranks its own fp64 logits; the GPU ranks its fp32 logits"}
    return base, indep


def measure(cfg, args, headline: bool, clock=None):
    """Every measurement of one layer; returns its per-config record."""
    import numpy as np
    import torch

    import mixture_experts_layer_15_amd as moe
    from mixture_experts_layer_15_amd import synthetic

    dev = synthetic.make_inputs(cfg, seed=0, device="cuda")
    x0 = dev["x"]
    xb = x0.numel() * x0.element_size()
    n_rot = max(1, min(64, -(-512 * 2 ** 20 // xb)))   # >= 512 MB of distinct token batches
    xs = [x0] + [x0.roll(i, dims=0).contiguous() for i in range(1, n_rot)]
    wr, bias, wg, wu, wd = dev["w_router"], dev["bias"], dev["w_gate"], dev["w_up"], dev["w_down"]

    R = moe.max_rows(cfg)
    dt = x0.dtype
    E = lambda shape, d=torch.float32: torch.empty(shape, dtype=d, device="cuda")
    logits, idx, gate = E((cfg.T, cfg.E)), E((cfg.T, cfg.k), torch.int32), E((cfg.T, cfg.k))
    x_perm = E((R, cfg.d), dt)
    count, offset = E(cfg.E, torch.int32), E(cfg.E + 1, torch.int32)
    row_of, tor = E((cfg.T, cfg.k), torch.int32), E(max(cfg.T * cfg.k, R), torch.int32)
    h, y_perm, y = E((R, cfg.d_ff), dt), E((R, cfg.d), dt), E((cfg.T, cfg.d), dt)
    dws = moe.workspace_bytes(cfg, dispatch_only=True)
    dsp_ws = torch.empty(max(dws, 16), dtype=torch.uint8, device="cuda")

    L = moe.lib()
    c = moe.cconfig(cfg)
    P = moe._ptr
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

    K, W = args.steps, args.warmup
    # the staged calls with events between the stages, first: at least 30
    # runs and at least a quarter second of GPU work, which also brings the
    # clocks up from idle before the fused steps are timed
    for i in range(W):
        step(xs[i % n_rot])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step(xs[0])
    torch.cuda.synchronize()
    est = max(time.perf_counter() - t0, 1e-5)
    ns = int(min(2000, max(30, K, 0.25 / est)))
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(ns)]
    for i in range(ns):
        step(xs[i % n_rot], evs[i])
    torch.cuda.synchronize()
    names = ["route", "dispatch", "gate_up", "down", "combine"]
    st = {n: [evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(ns)] for j, n in enumerate(names)}
    stage_med = {n: median(v) for n, v in st.items()}
    stage_mean = {n: float(np.mean(v)) for n, v in st.items()}

    # the fused entry point: W warmup steps, then exactly K steps between two
    # synchronisations give the step time (and, for the headline layer, `value`)
    fwd = moe.Forward(cfg)
    for i in range(W):
        fwd(xs[i % n_rot], wr, bias, wg, wu, wd, y)
    torch.cuda.synchronize()
    ctx = clock if (headline and clock is not None) else None
    if ctx:
        ctx.__enter__()
    t1 = time.perf_counter()
    for i in range(K):
        fwd(xs[i % n_rot], wr, bias, wg, wu, wd, y)
    torch.cuda.synchronize()
    fused_ms = (time.perf_counter() - t1) * 1e3 / K
    if ctx:
        ctx.__exit__(None, None, None)
    # the fused steps once more, each between two events, for their median
    nf = max(30, K)
    fe = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(nf)]
    for i in range(nf):
        fe[i][0].record()
        fwd(xs[i % n_rot], wr, bias, wg, wu, wd, y)
        fe[i][1].record()
    torch.cuda.synchronize()
    fused_ev = [a.elapsed_time(b) for a, b in fe]

    bwd_ms = None
    if cfg.dtype == "bf16" and not args.no_backward:
        dy = synthetic.make_dy(cfg, seed=1, device="cuda")
        bw = moe.Backward(cfg)
        bargs = (wr, bias, wg, wu, wd, dy)
        out = bw(xs[0], *bargs)
        for i in range(1, W):
            bw(xs[i % n_rot], *bargs, out=out)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(K):
            bw(xs[i % n_rot], *bargs, out=out)
        b.record()
        torch.cuda.synchronize()
        bwd_ms = a.elapsed_time(b) / K
        del out, bw, dy

    # variants of the layer on the same inputs (outside every timed region
    # above): the padded-capacity layout and the choice-order drop priority
    # (layers with a capacity limit and a fixed expert count), the MLP router at
    # the ZAYA1 page's widths (r = 256, m = 1024) on this layer's tokens, and
    # one step of its PID load-balance controller
    variants = None
    if not args.no_variants:
        variants = {}
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

        def timed(fn, n=10):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            ev0.record()
            for _ in range(n):
                fn()
            ev1.record()
            torch.cuda.synchronize()
            return ev0.elapsed_time(ev1) / n

        if cfg.cap_den > 0 and cfg.route_threshold == 0:
            yv = torch.empty_like(y)
            for key, vcfg in (("padded_layout_ms_per_step", cfg.scaled(layout=1)),
                              ("choice_order_ms_per_step", cfg.scaled(drop_policy=1))):
                fv = moe.Forward(vcfg)
                variants[key] = round(timed(lambda: fv(xs[0], wr, bias, wg, wu, wd, yv)), 4)
                del fv
            del yv
        if cfg.dtype == "bf16":
            g = torch.Generator(device="cuda").manual_seed(7)
            rnd = lambda *shape, sc: (torch.randn(*shape, generator=g, device="cuda") * sc).to(
                torch.bfloat16)
            r_, m_ = 256, 1024
            router = dict(w_down=rnd(cfg.d, r_, sc=cfg.d ** -0.5), w1=rnd(r_, m_, sc=r_ ** -0.5),
                          w2=rnd(m_, m_, sc=m_ ** -0.5), w3=rnd(m_, cfg.E, sc=m_ ** -0.5))
            prev = rnd(cfg.T, r_, sc=1.0)
            variants["mlp_router_ms"] = round(
                timed(lambda: moe.route_mlp(cfg, xs[0], prev, router, 0.5, 1e-6)), 4)
            del router, prev
        st_pid = torch.zeros((2, cfg.E), dtype=torch.float64, device="cuda")
        variants["pid_update_us_per_call"] = round(
            1e3 * timed(lambda: moe.pid_update(cfg, count, st_pid, 0.2, 0.02, 0.0), n=100), 2)
        torch.cuda.synchronize()

    # algorithmic work of the first batch's routing
    step(xs[0])
    torch.cuda.synchronize()
    ls = moe.load_stats(cfg, count).cpu().numpy()
    cnt = count.cpu().numpy()
    n_kept = int(offset.cpu().numpy()[-1])
    rows = row_of.cpu().numpy()
    idx_h = idx.cpu().numpy()
    active = int((rows >= 0).any(1).sum())
    a = algorithmic(cfg, cnt, n_kept, active)
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    gbs = lambda nbytes, ms: nbytes / (ms * 1e-3) / 1e9
    gemm_med = stage_med["gate_up"] + stage_med["down"]
    gemm_tf = (a["gate_up_flops"] + a["down_flops"]) / (gemm_med * 1e-3) / 1e12
    traffic, tkernel = measured_traffic(cfg)
    rec = {
        "workload": f"{cfg.name}: T={cfg.T} d={cfg.d} E={cfg.E} top-{cfg.k} GeGLU d_ff={cfg.d_ff} "
                    f"{cfg.dtype}",
        "T": cfg.T, "d": cfg.d, "E": cfg.E, "k": cfg.k, "d_ff": cfg.d_ff,
        "temperature": cfg.temperature,
        "capacity_factor": None if cfg.cap_den == 0 else cfg.cap_num / cfg.cap_den,
        "rows_kept": n_kept, "tokens_active": active,
        "tokens_per_s": round(cfg.T / (fused_ms * 1e-3), 1),
        "ms_per_step": round(fused_ms, 4),
        "fused_ms_median_events": round(median(fused_ev), 4),
        "stage_timings": ns,
        "stage_ms_median": {n: round(v, 4) for n, v in stage_med.items()},
        "stage_ms_mean": {n: round(v, 4) for n, v in stage_mean.items()},
        "grouped_gemm_tflops": round(gemm_tf, 1),
        "grouped_gemm_frac_of_mfma_peak": round(gemm_tf / peak, 4),
        "gate_up": {"tflops": round(a["gate_up_flops"] / (stage_med["gate_up"] * 1e-3) / 1e12, 1),
                    "frac_of_mfma_peak": round(a["gate_up_flops"] / (stage_med["gate_up"] * 1e-3)
                                               / 1e12 / peak, 4),
                    "frac_of_hbm_peak": round(gbs(a["gate_up_bytes"], stage_med["gate_up"])
                                              / PEAK_HBM_GBS, 4)},
        "down": {"tflops": round(a["down_flops"] / (stage_med["down"] * 1e-3) / 1e12, 1),
                 "frac_of_mfma_peak": round(a["down_flops"] / (stage_med["down"] * 1e-3)
                                            / 1e12 / peak, 4),
                 "frac_of_hbm_peak": round(gbs(a["down_bytes"], stage_med["down"])
                                           / PEAK_HBM_GBS, 4)},
        "route_gbs": round(gbs(a["route_bytes"], stage_med["route"]), 1),
        "dispatch_gbs": round(gbs(a["dispatch_bytes"], stage_med["dispatch"]), 1),
        "dispatch_frac_of_hbm_peak": round(gbs(a["dispatch_bytes"], stage_med["dispatch"])
                                           / PEAK_HBM_GBS, 4),
        "combine_gbs": round(gbs(a["combine_bytes"], stage_med["combine"]), 1),
        "combine_frac_of_hbm_peak": round(gbs(a["combine_bytes"], stage_med["combine"])
                                          / PEAK_HBM_GBS, 4),
        "algorithmic": {k2: (round(v) if isinstance(v, float) else v) for k2, v in a.items()},
        "expert_load": {"mean": round(float(ls[0]), 2), "max": int(ls[1]), "min": int(ls[2]),
                        "max_over_mean": round(float(ls[3]), 4),
                        "max_deviation": round(float(ls[4]), 4), "cv": round(float(ls[5]), 4),
                        "dropped": int(ls[6]), "empty_experts": int(ls[7])},
        "roofline": roofline(cfg, a, stage_mean["gate_up"], peak, traffic, tkernel),
        "variants": variants,
        "backward": None if bwd_ms is None else {
            "ms_per_step": round(bwd_ms, 4),
            "tokens_per_s": round(cfg.T / (bwd_ms * 1e-3), 1),
            # recomputed g and u (2), dh (1), dx_perm (2), three weight gradients (3):
            # 8 products of 2 n_kept d d_ff flops each
            "gemm_tflops": round(16 * n_kept * cfg.d * cfg.d_ff / (bwd_ms * 1e-3) / 1e12, 1),
            "gemm_frac_of_peak": round(16 * n_kept * cfg.d * cfg.d_ff / (bwd_ms * 1e-3) / 1e12
                                       / peak, 4)},
    }
    if cfg.zipf_bias is not None:
        rec["expert0_token_share"] = round(float((idx_h == 0).any(1).mean()), 4)
    if cfg.route_threshold > 0:
        kt = (idx_h >= 0).sum(1)
        rec["experts_per_token"] = {"k_min": cfg.k_min, "k_max": cfg.k,
                                    "threshold": cfg.route_threshold,
                                    "mean": round(float(kt.mean()), 4),
                                    "tokens_by_count": {str(j): int((kt == j).sum())
                                                        for j in range(cfg.k_min, cfg.k + 1)}}
    del xs, x_perm, h, y_perm, fwd
    torch.cuda.synchronize()
    if not args.no_cpu_baseline:
        host = {k2: (None if v is None else v.cpu()) for k2, v in dev.items()}
        target = args.cpu_seconds if headline else max(4.0, args.cpu_seconds / 2)
        rec["cpu_baseline"], rec["independent_logits"] = cpu_baseline(cfg, host, idx_h, rows,
                                                                      target)
        del host
    del dev
    torch.cuda.empty_cache()
    return rec


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "this layer's forward is measured on a single MI355X.", file=sys.stderr)
        sys.exit(2)

    import torch

    import mixture_experts_layer_15_amd as moe
    from mixture_experts_layer_15_amd import configs

    if args.copy_calibration:
        n = args.copy_calibration * 2 ** 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 5}), flush=True)
        return

    torch.cuda.set_device(0)
    L = moe.lib()
    probes = None if args.no_probes else run_probes(L, torch)
    clock = ClockSampler()
    head_cfg = configs.get(args.config)
    per = {head_cfg.name: measure(head_cfg, args, True, clock)}
    if not args.only_headline:
        for name in OTHERS:
            if name != head_cfg.name:
                per[name] = measure(configs.get(name), args, False)
        # the wide layer with the page's 2-4 experts per token (a variant)
        per["wide_dynamic"] = measure(configs.WIDE_DYNAMIC, args, False)
    hr = per[head_cfg.name]
    roof = dict(hr["roofline"])
    if probes and roof["unit"] == "TFLOP/s":
        roof["frac_of_measured_peak"] = round(roof["achieved"] /
                                              probes["mfma_bf16_tflops"]["median"], 4)
        if head_cfg.name == "longseq":
            roof["ratio_to_vendor_gemm"] = round(
                roof["achieved"] /
                probes["vendor_gemm_bf16"]["long_sequence_expert_gate_up"]["tflops"], 4)
    elif probes:
        roof["frac_of_measured_peak"] = round(roof["achieved"] / probes["hbm_copy_gbs"]["median"], 4)
    out = {
        "metric": METRIC,
        "value": hr["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": hr["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head_cfg.dtype,
        "data": "synthetic (seeded N(0,1) tokens, N(0,1/fan_in) random-init weights)",
        "config": {"workload": hr["workload"], "T": head_cfg.T, "d": head_cfg.d,
                   "E": head_cfg.E, "k": head_cfg.k, "d_ff": head_cfg.d_ff,
                   "temperature": head_cfg.temperature,
                   "capacity_factor": hr["capacity_factor"], "rows_kept": hr["rows_kept"],
                   "parallelism": "single GPU"},
        "grouped_gemm_tflops": hr["grouped_gemm_tflops"],
        "grouped_gemm_frac_of_peak": hr["grouped_gemm_frac_of_mfma_peak"],
        "stage_ms": hr["stage_ms_median"],
        "roofline": roof,
        "gpu_clock_during_timed_steps": clock.summary(),
        "probes": probes,
        "host": {"cpu_model": cpu_model(), "oracle_threads": oracle_threads()},
        "per_config": per,
    }
    if "cpu_baseline" in hr:
        out["cpu_baseline"] = hr["cpu_baseline"]
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

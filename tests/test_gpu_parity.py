"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Protocol: the oracle routes the GPU's exported fp32 logits (the layer makes
integer decisions -- top-k, drops, positions -- from fp32 logits, so both
sides decide from the same values); those decisions must match bit-exactly.
The logits themselves must sit within the fp32 summation bound of the
oracle's fp64 logits; floating outputs must satisfy
max |y - y*| / max |y*| <= 2e-2 (bf16 layers) or 1e-5 (fp32 layers).

Every output element is compared, on small shapes and on the five full-size
layers alike (those in the launch configuration the benchmark times): small
layers against the row-by-row C oracle, large ones against the by-expert
oracle (fp64 matrix products per expert).  Every output buffer starts as NaN
(floating) or -7 (integer), so an element no kernel writes fails."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_15_amd as moe
from mixture_experts_layer_15_amd import configs
from oracle import oracle as orc

from parity_util import (TOL_Y, bf16_ulp_distance, check_dispatch,
                         check_ffn_and_combine_by_expert, check_logits, check_route,
                         check_x_perm, expert_of_rows, fused_down_split, gpu_inputs, rel_err,
                         sample_rows, say, to_np)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()   # raises if the HIP library is missing


def run_layer(cfg, dev, host, full=True, seed=0, label=""):
    """Every stage through the C ABI, each checked against the oracle on every
    element: logits of every token, routing, dispatch, x_perm, every kept row
    of h and y_perm, y of every token, and the fused forward.  Small layers
    use the row-by-row C oracle; large ones the by-expert oracle (fp64 matrix
    products per expert block, pinned to the C oracle).  ``full=False`` keeps
    the old sampled check for callers that only want the integer outputs and
    a quick y check."""
    rng = np.random.default_rng(seed)
    x, wr, b = dev["x"], dev["w_router"], dev["bias"]
    say(f"[{label}] moe_route T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k}")
    logits, idx, gate = moe.route(cfg, x, wr, b)
    torch.cuda.synchronize()
    lg_h, idx_h, gate_h = logits.cpu(), idx.cpu(), gate.cpu()
    toks = np.arange(cfg.T) if full else np.unique(rng.integers(0, cfg.T, size=256))
    if cfg.T:
        check_logits(lg_h, host["x"], host["w_router"], host["bias"], toks)
    oidx, ogate, _ = check_route(cfg, lg_h, idx_h, gate_h)

    say(f"[{label}] moe_dispatch")
    dsp = moe.dispatch(cfg, idx, x)
    torch.cuda.synchronize()
    od = check_dispatch(cfg, oidx, dsp)
    n = od["n_kept"]
    check_x_perm(x, dsp["x_perm"], od["token_of_row"], n)

    say(f"[{label}] moe_expert_ffn rows={n}")
    h, y_perm = moe.expert_ffn(cfg, dsp["x_perm"], dsp["expert_offset"], dev["w_gate"],
                               dev["w_up"], dev["w_down"])
    torch.cuda.synchronize()
    rowwise = n * cfg.d * cfg.d_ff <= (1 << 28)
    ystar = None
    if full and not rowwise:
        ystar = check_ffn_and_combine_by_expert(cfg, host, od, ogate, h, y_perm, label)
    else:
        rows = sample_rows(od["offset"], n, full, rng)
        if rows.size:
            ex = expert_of_rows(od["offset"], rows)
            oh, oo = orc.ffn_rows(od["token_of_row"][rows], ex, host["x"], host["w_gate"],
                                  host["w_up"], host["w_down"], want_h=True)
            eh = rel_err(to_np(h[torch.from_numpy(rows).cuda()]), oh)
            eo = rel_err(to_np(y_perm[torch.from_numpy(rows).cuda()]), oo)
            say(f"[{label}] h err {eh:.3g}  y_perm err {eo:.3g} over {rows.size} rows")
            assert eh <= TOL_Y[cfg.dtype] and eo <= TOL_Y[cfg.dtype]

    say(f"[{label}] moe_combine")
    y = moe.combine(cfg, y_perm, dsp["row_of"], gate)
    torch.cuda.synchronize()
    stoks = np.arange(cfg.T)
    if cfg.T:
        row_of = od["row_of"]
        if ystar is None:
            if not full:
                dropped = np.nonzero((row_of < 0).any(1))[0]
                stoks = np.unique(np.concatenate([rng.integers(0, cfg.T, size=48),
                                                  dropped[:16], [0, cfg.T - 1]]))
            ofw = orc.forward(host["x"], host["w_router"], host["bias"], host["w_gate"],
                              host["w_up"], host["w_down"], k=cfg.k,
                              tau=float(np.float32(cfg.temperature)),
                              renormalize=cfg.renormalize, cap_num=cfg.cap_num,
                              cap_den=cfg.cap_den, drop_policy=cfg.drop_policy,
                              logits_in=lg_h.double().numpy(), tokens=stoks,
                              k_min=cfg.k_min,
                              threshold=float(np.float32(cfg.route_threshold)))
            ystar = ofw["y"]
        ey = rel_err(to_np(y[torch.from_numpy(stoks).cuda()]), ystar)
        say(f"[{label}] y err {ey:.3g} over {stoks.size} tokens")
        assert ey <= TOL_Y[cfg.dtype]
        fully = (row_of < 0).all(1)
        if fully.any():   # tokens with every assignment dropped are exactly zero
            zt = torch.from_numpy(np.nonzero(fully)[0]).cuda()
            assert (y.index_select(0, zt).float() == 0).all()

    say(f"[{label}] moe_forward")
    yf = moe.forward(cfg, x, wr, b, dev["w_gate"], dev["w_up"], dev["w_down"])
    torch.cuda.synchronize()
    iv = torch.int16 if y.dtype == torch.bfloat16 else torch.int32
    if fused_down_split(cfg):
        # the fused down GEMM sums K in two fp32 slices: the outputs differ from
        # the staged calls' only by that summation order -- a rounding step at
        # most, measured against the output's scale (near-cancelling values can
        # differ by many of their own ulps) -- and meet the oracle's tolerance
        d_fs = rel_err(to_np(yf), to_np(y))
        e_f = rel_err(to_np(yf[torch.from_numpy(stoks).cuda()]), ystar) if cfg.T else 0.0
        say(f"[{label}] fused forward: {d_fs:.3g} of max |y| from the staged calls "
            f"({bf16_ulp_distance(yf, y)} ulp at most), y err {e_f:.3g}")
        assert d_fs <= 2.0 ** -7 and e_f <= TOL_Y[cfg.dtype]
    else:
        assert torch.equal(yf.view(iv), y.view(iv)), "fused forward differs from the staged calls"
    return dict(logits=logits, idx=idx, gate=gate, dsp=dsp, h=h, y_perm=y_perm, y=y, n=n,
                oidx=oidx, ogate=ogate, od=od)


SMALL = [
    # ragged tails everywhere: T % 64, d % 128 == 64, E % 8 != 0, k = 3, heavy drops, bias
    ("ragged", configs.get("tiny").scaled(T=1000, d=192, E=5, k=3, d_ff=320, temperature=0.5,
                                          cap_num=1, cap_den=1, renormalize=True, dtype="bf16",
                                          zipf_bias=1.2)),
    ("single", configs.get("tiny").scaled(T=1, d=64, E=1, k=1, d_ff=64, dtype="bf16")),
    ("maxEk", configs.get("tiny").scaled(T=300, d=256, E=256, k=8, d_ff=128, cap_num=5,
                                         cap_den=4, renormalize=True, dtype="bf16")),
    ("zero_capacity", configs.get("tiny").scaled(T=4096, d=128, E=8, k=2, d_ff=192, cap_num=0,
                                                 cap_den=1, renormalize=True, dtype="bf16")),
    ("f32_ragged", configs.get("tiny").scaled(T=777, d=128, E=6, k=2, d_ff=192, temperature=0.7,
                                              cap_num=3, cap_den=2, renormalize=True)),
    ("many_chunks", configs.get("tiny").scaled(T=70000, d=64, E=16, k=2, d_ff=64, cap_num=5,
                                               cap_den=4, renormalize=True, dtype="bf16")),
    ("tiles_2x", configs.get("tiny").scaled(T=2500, d=384, E=3, k=1, d_ff=448, dtype="bf16")),
    # k = E: every expert chosen, renormalised gates = the softmax over all experts
    ("k_eq_E", configs.get("tiny").scaled(T=500, d=128, E=4, k=4, d_ff=128, temperature=0.5,
                                          renormalize=True, dtype="bf16")),
    # experts of very different sizes: 15 to 4054 rows on 256-row tiles (top-2,
    # 1365 rows per expert on average), 1 to 1868 rows on 640-row tiles (top-1,
    # 410 on average), and on 320-row tiles (top-1, 256 on average) with the
    # hot experts over several M-tiles
    ("skew_256", configs.get("tiny").scaled(T=4096, d=128, E=6, k=2, d_ff=192, temperature=0.5,
                                            renormalize=True, dtype="bf16", zipf_bias=2.5)),
    ("skew_640_top1", configs.get("tiny").scaled(T=2048, d=128, E=5, k=1, d_ff=192,
                                                 temperature=0.5, dtype="bf16", zipf_bias=3.0)),
    ("skew_320", configs.get("tiny").scaled(T=1536, d=128, E=6, k=1, d_ff=192, temperature=0.5,
                                            dtype="bf16", zipf_bias=2.5)),
    # 320-640 rows per expert on average: 640-row tiles, with skew so that the
    # hot experts take two or more of them and the cold ones a few rows
    ("skew_640", configs.get("tiny").scaled(T=2000, d=192, E=8, k=2, d_ff=320, temperature=0.5,
                                            renormalize=True, dtype="bf16", zipf_bias=2.0)),
    # the validation limits: d = 16384 (router and gate/up K of 16384, down N of 16384) with
    # the smallest d_ff (one ragged gate/up N-tile); d_ff = 65536 (down K of 65536, fused
    # two-K-slice down GEMM) with the smallest d; the same d in fp32; E = 256 with k = 8 on
    # the multi-block dispatch
    ("max_d", configs.get("tiny").scaled(T=300, d=16384, E=4, k=2, d_ff=64, temperature=0.5,
                                         renormalize=True, dtype="bf16")),
    ("max_dff", configs.get("tiny").scaled(T=200, d=64, E=2, k=1, d_ff=65536, dtype="bf16")),
    ("max_d_f32", configs.get("tiny").scaled(T=100, d=16384, E=3, k=1, d_ff=128)),
    ("max_Ek_blocks", configs.get("tiny").scaled(T=3000, d=64, E=256, k=8, d_ff=64, cap_num=5,
                                                 cap_den=4, renormalize=True, dtype="bf16")),
    # top-1, every token kept, few experts: the fused forward's down GEMM in two
    # K slices (d = 320: a ragged second N-tile)
    ("split_down", configs.get("tiny").scaled(T=3000, d=320, E=6, k=1, d_ff=384,
                                              temperature=0.7, dtype="bf16")),
    # more than 512 rows per expert on average: 256-row tiles, and the experts
    # under 64 rows in their own launch of 128-row tiles (7 and 2 rows here)
    ("few_rows_split", configs.get("tiny").scaled(T=12288, d=128, E=5, k=1, d_ff=192,
                                                  temperature=0.5, dtype="bf16", zipf_bias=3.0)),
]


@pytest.mark.parametrize("name,cfg", SMALL, ids=[s[0] for s in SMALL])
def test_small_layers_every_element(name, cfg):
    dev, host = gpu_inputs(cfg, seed=3)
    run_layer(cfg, dev, host, full=True, seed=3, label=name)


def test_hot_expert_overflow():
    """Every token's first choice is expert 0 (large bias): capacity drops in
    token order decide almost everything."""
    cfg = configs.get("tiny").scaled(T=3000, d=128, E=6, k=2, d_ff=128, cap_num=5, cap_den=4,
                                     renormalize=True, dtype="bf16", temperature=0.3)
    dev, host = gpu_inputs(cfg, seed=4)
    bias = torch.tensor([30.0, 0, 0, 0, 0, 0], dtype=torch.float32)
    dev["bias"], host["bias"] = bias.cuda(), bias
    out = run_layer(cfg, dev, host, full=True, seed=4, label="hot")
    C = orc.capacity(cfg.T, cfg.E, cfg.k, 5, 4)
    assert int(out["dsp"]["expert_count"][0]) == cfg.T
    assert int(out["dsp"]["expert_offset"][1]) == C


def test_empty_batch():
    cfg = configs.get("tiny").scaled(T=0, dtype="bf16", d=128, d_ff=128)
    dev, host = gpu_inputs(cfg.scaled(T=1))
    x = dev["x"][:0]
    logits, idx, gate = moe.route(cfg, x, dev["w_router"], None)
    dsp = moe.dispatch(cfg, idx, x)
    h, yp = moe.expert_ffn(cfg, dsp["x_perm"], dsp["expert_offset"], dev["w_gate"], dev["w_up"],
                           dev["w_down"])
    y = moe.combine(cfg, yp, dsp["row_of"], gate)
    yf = moe.forward(cfg, x, dev["w_router"], None, dev["w_gate"], dev["w_up"], dev["w_down"])
    torch.cuda.synchronize()
    assert y.shape == (0, cfg.d) and yf.shape == (0, cfg.d)
    assert (dsp["expert_offset"].cpu() == 0).all() and (dsp["expert_count"].cpu() == 0).all()


def test_route_from_logits_ties_and_signed_zero():
    T, E = 64, 20
    lg = torch.zeros((T, E), dtype=torch.float32)
    lg[1] = torch.arange(E, dtype=torch.float32) % 3          # repeated values
    lg[2, :] = -0.0
    lg[2, 7] = 0.0
    lg[3] = 1e30
    lg[3, 5] = -1e30
    lg[4] = torch.tensor([1.0, 1.0 + 2 ** -23] * 10)          # one-ulp differences
    lg[5:] = torch.randint(-2, 3, (T - 5, E)).float()         # many exact ties
    for k, tau, renorm in [(1, 1.0, False), (3, 0.3, True), (8, 2.0, True), (20, 1.0, True)]:
        cfg = configs.get("tiny").scaled(T=T, E=E, k=min(k, 8), temperature=tau,
                                         renormalize=renorm)
        if k > 8:
            continue
        idx, gate = moe.route_from_logits(cfg, lg.cuda())
        torch.cuda.synchronize()
        # row 3 has |l| = 1e30: exp underflows to exactly 0 for the far experts
        check_route(cfg, lg, idx.cpu(), gate.cpu())


def test_deterministic_reruns():
    cfg = configs.get("tiny").scaled(T=5000, d=256, E=12, k=2, d_ff=384, cap_num=5, cap_den=4,
                                     renormalize=True, dtype="bf16", temperature=0.3)
    dev, _ = gpu_inputs(cfg, seed=5)
    f = moe.Forward(cfg)
    a = f(dev["x"], dev["w_router"], None, dev["w_gate"], dev["w_up"], dev["w_down"]).clone()
    b = f(dev["x"], dev["w_router"], None, dev["w_gate"], dev["w_up"], dev["w_down"]).clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("name", [c.name for c in configs.CONFIGS])
def test_full_size_layer(name):
    """The five layers at their real sizes, in the launch configuration the
    benchmark times, every output element against the oracle."""
    cfg = configs.get(name)
    dev, host = gpu_inputs(cfg, seed=0)
    out = run_layer(cfg, dev, host, full=True, seed=0, label=name)
    cnt = out["dsp"]["expert_count"].cpu().numpy()
    say(f"[{name}] rows kept {out['n']} of {cfg.T * cfg.k}; largest expert share of "
        f"assignments {cnt.max() / max(cnt.sum(), 1):.3f}")
    if name == "skewed":
        share = float((out["oidx"] == 0).any(1).mean())
        say(f"[skewed] tokens with expert 0 among their choices: {share:.3f}")
        assert 0.25 <= share <= 0.35

"""GPU parity of the routing variants against the fp64 oracle, through the C ABI:
the choice-order drop priority (every first choice before every second
choice) and the expert-load telemetry.  Integer outputs bit-exact; the layer
output within the same tolerance as the main parity tests."""
import ctypes

import numpy as np
import pytest
import torch

import mixture_experts_layer_15_amd as moe
from mixture_experts_layer_15_amd import configs
from oracle import oracle as orc

from parity_util import (TOL_Y, check_route, gpu_inputs, oracle_capacity, rel_err, say,
                         to_np)
from test_gpu_parity import run_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


SMALL = configs.get("tiny").scaled(dtype="bf16", temperature=0.3, renormalize=True,
                                   cap_num=5, cap_den=4, drop_policy=1)
CHOICE_CASES = {
    # one-launch dispatch (T*k <= 16384), every output compared
    "choice_small": SMALL.scaled(T=1500, d=128, E=12, k=3, d_ff=192),
    # hot expert: Zipf bias, most assignments dropped
    "choice_hot": SMALL.scaled(T=3000, d=128, E=16, k=2, d_ff=128, zipf_bias=1.2),
    # multi-block histogram / scan / place path
    "choice_blocks": SMALL.scaled(T=20000, d=128, E=64, k=2, d_ff=128),
}


@pytest.mark.parametrize("name", list(CHOICE_CASES))
def test_choice_order_layer(name):
    cfg = CHOICE_CASES[name]
    dev, host = gpu_inputs(cfg, seed=3)
    run_layer(cfg, dev, host, full=True, seed=3, label=name)


def test_choice_order_full_size_skewed():
    cfg = configs.get("skewed").scaled(drop_policy=1)
    dev, host = gpu_inputs(cfg, seed=0)
    out = run_layer(cfg, dev, host, full=True, seed=0, label="skewed/choice")
    # the two priorities keep different assignment sets on this layer
    C = orc.capacity(cfg.T, cfg.E, cfg.k, cfg.cap_num, cfg.cap_den)
    tok = orc.dispatch(out["idx"].cpu().numpy(), cfg.E, C, 0)
    cho = orc.dispatch(out["idx"].cpu().numpy(), cfg.E, C, 1)
    say(f"[skewed/choice] kept {cho['n_kept']} (token order {tok['n_kept']}), "
        f"assignments kept by one order only: "
        f"{int(((tok['row_of'] >= 0) != (cho['row_of'] >= 0)).sum())}")
    assert ((tok["row_of"] >= 0) != (cho["row_of"] >= 0)).any()


@pytest.mark.parametrize("name,policy", [("zaya1", 0), ("skewed", 0), ("skewed", 1), ("wide", 0)])
def test_load_stats_match_oracle(name, policy):
    cfg = configs.get(name).scaled(drop_policy=policy)
    dev, _ = gpu_inputs(cfg, seed=0)
    _, idx, _ = moe.route(cfg, dev["x"], dev["w_router"], dev["bias"])
    dsp = moe.dispatch(cfg, idx, dev["x"])
    st = moe.load_stats(cfg, dsp["expert_count"])
    torch.cuda.synchronize()
    got = st.cpu().numpy()
    C = orc.capacity(cfg.T, cfg.E, cfg.k, cfg.cap_num, cfg.cap_den)
    want = orc.load_stats(dsp["expert_count"].cpu().numpy(), C)
    say(f"[{name}/{policy}] load: mean {want[0]:.1f} max/mean {want[3]:.3f} "
        f"max deviation {100 * want[4]:.1f}% CV {want[5]:.3f} dropped {int(want[6])} "
        f"empty {int(want[7])}")
    # counts, sums and the max/min-based ratios are exact in fp64; the CV sums
    # its squares in another order
    np.testing.assert_array_equal(got[[0, 1, 2, 3, 4, 6, 7]], want[[0, 1, 2, 3, 4, 6, 7]])
    assert abs(got[5] - want[5]) <= 1e-12 * max(1.0, abs(want[5]))


def test_load_stats_edge_counts():
    cfg = configs.get("tiny").scaled(E=256, k=1, cap_num=1, cap_den=2)
    for counts in (np.zeros(256, np.int32), np.r_[np.full(255, 0), 777].astype(np.int32),
                   np.arange(256, dtype=np.int32)):
        st = moe.load_stats(cfg, torch.from_numpy(counts).cuda())
        torch.cuda.synchronize()
        C = orc.capacity(cfg.T, cfg.E, cfg.k, cfg.cap_num, cfg.cap_den)
        want = orc.load_stats(counts, C)
        np.testing.assert_allclose(st.cpu().numpy(), want, rtol=1e-12, atol=0)


# ---------------------------------------------------------------- PID controller
# The MLP router's load-balance controller (one PID loop per expert on the
# relative load error, output the additive logit bias): fp64 on both sides,
# every operation rounded once in the same order, so the state must match the
# oracle exactly and the fp32 bias is the oracle's value rounded once.
@pytest.mark.parametrize("E", [1, 5, 64, 256])
def test_pid_controller_matches_the_oracle(E):
    cfg = configs.get("tiny").scaled(E=E, k=1)
    rng = np.random.default_rng(E)
    st_dev = torch.zeros((2, E), dtype=torch.float64, device="cuda")
    st_orc = np.zeros((2, E))
    say(f"[pid E={E}] six steps of moe_pid_update")
    for step in range(6):
        if step == 3:
            cnt = np.zeros(E, np.int32)                     # no assignments at all
        else:
            cnt = rng.integers(0, 3000, E).astype(np.int32)
            cnt[rng.integers(0, E)] = 0                     # an idle expert
        kp, ki, kd = rng.uniform(0, 1, 3)
        scale = min(1.0, (step + 1) / 4)
        bias = moe.pid_update(cfg, torch.from_numpy(cnt).cuda(), st_dev, kp, ki, kd, scale)
        st_orc, b_orc = orc.pid_update(cnt, st_orc, kp, ki, kd, scale)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(st_dev.cpu().numpy(), st_orc)
        np.testing.assert_array_equal(bias.cpu().numpy(), b_orc.astype(np.float32))


def test_pid_controller_closed_loop_on_the_gpu_router():
    """The controller fed back through the layer's own router and dispatch:
    a Zipf-skewed top-2 routing (about 30% of tokens choose expert 0) evens
    out, and every step's controller output equals the oracle's."""
    cfg = configs.get("skewed").scaled(T=8192, d=256, d_ff=64)
    dev, _ = gpu_inputs(cfg, seed=0)
    E = cfg.E
    st_dev = torch.zeros((2, E), dtype=torch.float64, device="cuda")
    st_orc = np.zeros((2, E))
    base = dev["bias"].clone()
    pid = torch.zeros(E, dtype=torch.float32, device="cuda")
    cv = []
    say("[pid loop] 80 steps of route, dispatch, moe_pid_update")
    for step in range(80):
        _, idx, _ = moe.route(cfg, dev["x"], dev["w_router"], base + pid)
        cnt = moe.dispatch(cfg, idx, dev["x"])["expert_count"]
        c = cnt.cpu().numpy()
        cv.append(float(c.std() / c.mean()))
        scale = min(1.0, (step + 1) / 10)
        pid = moe.pid_update(cfg, cnt, st_dev, 0.2, 0.02, 0.0, scale)
        st_orc, b_orc = orc.pid_update(c, st_orc, 0.2, 0.02, 0.0, scale)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(pid.cpu().numpy(), b_orc.astype(np.float32))
    say(f"[pid loop] load CV (std / mean): step 0 {cv[0]:.3f}, step 79 {cv[-1]:.3f}")
    assert cv[0] > 1.0 and cv[-1] < 0.15, cv


# ---------------------------------------------------------------- MLP router
# Logits of a bf16 network (four intermediate roundings): compared with the
# R13 metric at the layer's bf16 tolerance; the top-k and gates then follow the
# same-fp32-logits protocol as the linear router.
TOL_MLP_LOGITS = 2e-2


def _mlp_router_inputs(cfg, r, m, seed):
    g = torch.Generator().manual_seed(seed)
    n = lambda *s, sc=1.0: (torch.randn(*s, generator=g) * sc)
    bf = lambda t: t.to(torch.bfloat16)
    host = dict(w_down=bf(n(cfg.d, r, sc=cfg.d ** -0.5)), b_down=n(r, sc=0.1),
                w1=bf(n(r, m, sc=r ** -0.5)), b1=n(m, sc=0.1),
                w2=bf(n(m, m, sc=m ** -0.5)), b2=n(m, sc=0.1),
                w3=bf(n(m, cfg.E, sc=m ** -0.5)), b3=n(cfg.E, sc=0.1),
                pid_bias=n(cfg.E, sc=0.05))
    prev = bf(n(cfg.T, r))
    return host, prev


MLP_CASES = {
    "mlp_small": (configs.get("tiny").scaled(T=300, d=128, E=16, k=2, dtype="bf16",
                                             renormalize=True, temperature=0.3), 64, 128, True),
    "mlp_ragged": (configs.get("tiny").scaled(T=1001, d=192, E=24, k=3, dtype="bf16",
                                              renormalize=True), 128, 192, True),
    # the page's widths on the ZAYA1-like layer
    "mlp_zaya1": (configs.get("zaya1"), 256, 1024, False),
}


@pytest.mark.parametrize("name", list(MLP_CASES))
def test_mlp_router_matches_oracle(name):
    from parity_util import check_route, rel_err
    cfg, r, m, with_prev = MLP_CASES[name]
    dev_in, _ = gpu_inputs(cfg, seed=7)
    x = dev_in["x"]
    host, prev = _mlp_router_inputs(cfg, r, m, seed=11)
    rt = {k: v.cuda() for k, v in host.items()}
    prev_d = prev.cuda() if with_prev else None
    gamma, eps = 0.5, 1e-6
    say(f"[{name}] moe_route_mlp T={cfg.T} d={cfg.d} r={r} m={m} E={cfg.E} k={cfg.k}")
    lg, idx, gate = moe.route_mlp(cfg, x, prev_d, rt, gamma, eps)
    torch.cuda.synchronize()
    toks = np.arange(cfg.T)
    want = orc.mlp_router(x.cpu()[toks], prev[toks] if with_prev else None, gamma, eps,
                          host["w_down"], host["b_down"], host["w1"], host["b1"], host["w2"],
                          host["b2"], host["w3"], host["b3"], host["pid_bias"])["logits"]
    err = rel_err(lg.cpu().double().numpy()[toks], want)
    say(f"[{name}] logits err {err:.3g} over {toks.size} tokens")
    assert err <= TOL_MLP_LOGITS
    check_route(cfg, lg.cpu(), idx.cpu(), gate.cpu())
    # the same logits through the linear router's top-k entry point
    idx2, gate2 = moe.route_from_logits(cfg, lg)
    torch.cuda.synchronize()
    assert torch.equal(idx2, idx) and torch.equal(gate2, gate)


PADDED_CASES = {
    # top-2 renormalised, capacity 5/4, experts not a multiple of 8
    "padded_small": SMALL.scaled(T=1500, d=128, E=12, k=3, d_ff=192, drop_policy=0),
    # choice order, hot expert (Zipf bias): most slots of the cold experts empty
    "padded_hot": SMALL.scaled(T=3000, d=128, E=16, k=2, d_ff=128, zipf_bias=1.2),
    # top-1 with capacity 1/2: many drops, every expert full
    "padded_drops": SMALL.scaled(T=2000, d=192, E=8, k=1, d_ff=320, cap_num=1, cap_den=2,
                                 renormalize=False, drop_policy=0),
}


def _check_padded(cfg, dev, host, full, label):
    """Padded layout: dispatch maps bit-exact against the oracle's padded
    layout, empty rows zero, and the layer output bit-identical to the
    compact layout's (same rows, same per-row arithmetic)."""
    pad = cfg.scaled(layout=1)
    logits, idx, gate = moe.route(pad, dev["x"], dev["w_router"], dev["bias"])
    torch.cuda.synchronize()
    oidx, _, _ = check_route(pad, logits.cpu(), idx.cpu(), gate.cpu())
    C = min(orc.capacity(cfg.T, cfg.E, cfg.k, cfg.cap_num, cfg.cap_den), cfg.T)
    say(f"[{label}] moe_dispatch padded: E={cfg.E} C={C} rows={cfg.E * C}")
    dsp = moe.dispatch(pad, idx, dev["x"])
    torch.cuda.synchronize()
    od = orc.dispatch(oidx, cfg.E, C, cfg.drop_policy, layout=1)
    np.testing.assert_array_equal(dsp["expert_count"].cpu().numpy(), od["count"])
    np.testing.assert_array_equal(dsp["expert_offset"].cpu().numpy(), od["offset"])
    np.testing.assert_array_equal(dsp["row_of"].cpu().numpy(), od["row_of"])
    tor = dsp["token_of_row"].cpu().numpy()
    np.testing.assert_array_equal(tor[:od["n_rows"]], od["token_of_row"])
    assert (tor[od["n_rows"]:] == -1).all()
    xp = dsp["x_perm"]
    kept = torch.from_numpy(np.nonzero(od["token_of_row"] >= 0)[0]).cuda()
    empty = torch.from_numpy(np.nonzero(od["token_of_row"] < 0)[0]).cuda()
    src = torch.from_numpy(od["token_of_row"][od["token_of_row"] >= 0].astype(np.int64)).cuda()
    assert torch.equal(xp.index_select(0, kept).view(torch.int16),
                       dev["x"].index_select(0, src).view(torch.int16))
    if empty.numel():
        assert (xp.index_select(0, empty).float() == 0).all()
    say(f"[{label}] kept {od['n_kept']} of {od['n_rows']} padded rows")
    say(f"[{label}] moe_forward padded vs compact")
    args = (dev["x"], dev["w_router"], dev["bias"], dev["w_gate"], dev["w_up"], dev["w_down"])
    y_pad = moe.forward(pad, *args)
    y_cmp = moe.forward(cfg, *args)
    torch.cuda.synchronize()
    assert torch.equal(y_pad.view(torch.int16), y_cmp.view(torch.int16)), \
        "padded and compact layouts give different outputs"
    if full:
        ofw = orc.forward(host["x"], host["w_router"], host["bias"], host["w_gate"],
                          host["w_up"], host["w_down"], k=cfg.k,
                          tau=float(np.float32(cfg.temperature)), renormalize=cfg.renormalize,
                          cap_num=cfg.cap_num, cap_den=cfg.cap_den, drop_policy=cfg.drop_policy,
                          logits_in=logits.cpu().double().numpy())
        err = rel_err(to_np(y_pad), ofw["y"])
        say(f"[{label}] y err {err:.3g}")
        assert err <= TOL_Y[cfg.dtype]


@pytest.mark.parametrize("name", list(PADDED_CASES))
def test_padded_layout(name):
    cfg = PADDED_CASES[name]
    dev, host = gpu_inputs(cfg, seed=5)
    _check_padded(cfg, dev, host, full=True, label=name)


def test_padded_layout_full_size_skewed():
    cfg = configs.get("skewed")
    dev, host = gpu_inputs(cfg, seed=0)
    _check_padded(cfg, dev, host, full=False, label="skewed/padded")


# ---------------------------------------------------------------- dynamic expert count
# each token takes k_min .. k experts: the fewest whose softmax mass reaches the
# threshold (the TorchTitan 1K-GPU article's 2-4 experts per token, section 2.1)
DYN = configs.get("tiny").scaled(dtype="bf16", renormalize=True, cap_num=5, cap_den=4,
                                 k=4, k_min=2, route_threshold=0.6)
DYN_CASES = {
    # one-launch dispatch path, temperature 0.3 as on the page's layer
    "dyn_small": DYN.scaled(T=2000, d=128, E=16, d_ff=192, temperature=0.3),
    # multi-block dispatch path, ragged token count, capacity factor 1 (drops)
    "dyn_blocks": DYN.scaled(T=9001, d=128, E=24, d_ff=128, temperature=0.5, cap_num=1,
                             cap_den=1),
    # choice-order drops, raw gates, k_min 1 up to 3 experts
    "dyn_choice_raw": DYN.scaled(T=6000, d=64, E=10, k=3, k_min=1, route_threshold=0.8,
                                 d_ff=128, renormalize=False, drop_policy=1),
    # no capacity limit, threshold 1: every token takes all k
    "dyn_all": DYN.scaled(T=700, d=64, E=6, d_ff=64, cap_num=0, cap_den=0,
                          route_threshold=1.0),
}


@pytest.mark.parametrize("name", list(DYN_CASES))
def test_dynamic_expert_count_layer(name):
    cfg = DYN_CASES[name]
    dev, host = gpu_inputs(cfg, seed=8)
    out = run_layer(cfg, dev, host, full=True, seed=8, label=name)
    kt = (out["oidx"] >= 0).sum(1)
    assert kt.min() >= cfg.k_min and kt.max() <= cfg.k
    if name == "dyn_all":
        assert (kt == cfg.k).all()
    else:
        assert len(set(kt.tolist())) > 1, "every token took the same number of experts"


def test_dynamic_expert_count_full_size_wide():
    """The page's layer (128 experts, capacity factor 1.25, temperature 0.3)
    with 2-4 experts per token, at full size, every output element."""
    cfg = configs.WIDE_DYNAMIC
    dev, host = gpu_inputs(cfg, seed=0)
    out = run_layer(cfg, dev, host, full=True, seed=0, label="wide_dynamic")
    kt = (out["oidx"] >= 0).sum(1)
    say(f"[wide_dynamic] tokens taking 2/3/4 experts: "
        f"{np.bincount(kt, minlength=5)[2:].tolist()}, capacity "
        f"{oracle_capacity(cfg, out['oidx'])}, rows kept {out['n']}")
    assert kt.min() >= 2 and kt.max() <= 4
    st = moe.load_stats(cfg, out["dsp"]["expert_count"])
    torch.cuda.synchronize()
    want = orc.load_stats(out["dsp"]["expert_count"].cpu().numpy(),
                          oracle_capacity(cfg, out["oidx"]))
    got = st.cpu().numpy()
    np.testing.assert_array_equal(got[[0, 1, 2, 3, 4, 6, 7]], want[[0, 1, 2, 3, 4, 6, 7]])

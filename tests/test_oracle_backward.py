"""Pins of the oracle's backward pass (gradients of the layer for an upstream
dy) to things other than itself: central finite differences of the oracle's
own forward in fp64 (fp32 inputs perturbed by exactly representable steps),
the softmax backward's zero sum, the cases with no router gradient (one
expert) or no gradient at all (capacity 0), exact linearity in dy, and bf16
inputs giving the gradients of the same values held in fp32.  The routing
(top-k, drops) is piecewise constant: perturbations that flip it are skipped
and counted."""
import numpy as np
import pytest
import torch

from oracle import oracle as orc

NAMES = [("x", "dx"), ("w_router", "dw_router"), ("bias", "dbias"), ("w_gate", "dw_gate"),
         ("w_up", "dw_up"), ("w_down", "dw_down")]


def _layer(T, d, E, d_ff, seed, dtype=torch.float32):
    g = torch.Generator().manual_seed(seed)
    r = lambda *s, sc=1.0: (torch.randn(*s, generator=g) * sc).to(dtype)
    return dict(x=r(T, d), w_router=r(d, E), bias=r(E, sc=0.5).float(), w_gate=r(E, d, d_ff, sc=0.7),
                w_up=r(E, d, d_ff, sc=0.7), w_down=r(E, d_ff, d, sc=0.7))


def _loss(p, dy, kw):
    f = orc.forward(p["x"], p["w_router"], p["bias"], p["w_gate"], p["w_up"], p["w_down"], **kw)
    return float((f["y"] * dy).sum()), f["idx"], f["row_of"]


def _fd_check(p, dy, kw, h=2.0 ** -10, rtol=2e-4):
    got = orc.backward(p["x"], p["w_router"], p["bias"], p["w_gate"], p["w_up"], p["w_down"], dy,
                       **kw)
    _, idx0, row0 = _loss(p, dy, kw)
    skipped = checked = 0
    for name, gname in NAMES:
        t = p[name]
        g = got[gname]
        scale = np.abs(g).max() + 1e-30
        for flat in range(t.numel()):
            ix = np.unravel_index(flat, tuple(t.shape))
            q = dict(p)
            tp, tm = t.clone(), t.clone()
            tp[ix] += h
            tm[ix] -= h
            q[name] = tp
            lp, ip, rp = _loss(q, dy, kw)
            q[name] = tm
            lm, im, rm = _loss(q, dy, kw)
            if not ((ip == idx0).all() and (im == idx0).all() and (rp == row0).all()
                    and (rm == row0).all()):
                skipped += 1
                continue
            dp = float(tp[ix].double() - t[ix].double())
            dm = float(tm[ix].double() - t[ix].double())
            fd = (lp - lm) / (dp - dm)
            assert abs(fd - g[ix]) <= rtol * max(abs(fd), 1e-2 * scale), \
                f"{gname}{ix}: finite difference {fd} vs {g[ix]}"
            checked += 1
    assert skipped <= checked // 20, f"{skipped} perturbations flipped the routing"
    return got


@pytest.mark.parametrize("k,renorm,cap", [(1, False, (0, 0)), (2, True, (0, 0)),
                                          (2, True, (1, 2)), (3, False, (3, 4))])
def test_gradients_match_finite_differences(k, renorm, cap):
    T, d, E, d_ff = 7, 6, 4, 5
    p = _layer(T, d, E, d_ff, seed=10 * k + int(renorm))
    dy = torch.randn((T, d), generator=torch.Generator().manual_seed(99)).double().numpy()
    kw = dict(k=k, tau=0.7, renormalize=renorm, cap_num=cap[0], cap_den=cap[1])
    got = _fd_check(p, dy, kw)
    if cap == (1, 2):   # C = ceil(k T / 2E) = 2: some assignments dropped
        assert (got["row_of"] < 0).any()


def test_choice_order_gradients_match_finite_differences():
    T, d, E, d_ff = 8, 4, 3, 4
    p = _layer(T, d, E, d_ff, seed=5)
    dy = torch.randn((T, d), generator=torch.Generator().manual_seed(7)).double().numpy()
    kw = dict(k=2, tau=1.3, renormalize=True, cap_num=3, cap_den=4, drop_policy=1)
    _fd_check(p, dy, kw)


def _grads(p, dy, **kw):
    return orc.backward(p["x"], p["w_router"], p["bias"], p["w_gate"], p["w_up"], p["w_down"],
                        dy, **kw)


def test_softmax_backward_sums_to_zero_and_single_expert_has_no_router_gradient():
    p = _layer(20, 8, 6, 8, seed=3)
    dy = np.random.default_rng(0).standard_normal((20, 8))
    g = _grads(p, dy, k=2, tau=0.5, renormalize=True, cap_num=0, cap_den=0)
    assert abs(g["dbias"].sum()) <= 1e-12 * np.abs(g["dbias"]).sum()
    p1 = _layer(20, 8, 1, 8, seed=4)
    g1 = _grads(p1, dy, k=1, tau=1.0, renormalize=False, cap_num=0, cap_den=0)
    assert (g1["dw_router"] == 0).all() and (g1["dbias"] == 0).all()


def test_zero_capacity_has_zero_gradients():
    p = _layer(10, 4, 3, 4, seed=6)
    dy = np.random.default_rng(1).standard_normal((10, 4))
    g = _grads(p, dy, k=2, tau=1.0, renormalize=True, cap_num=0, cap_den=1)
    for _, gname in NAMES:
        assert (g[gname] == 0).all(), gname


def test_linear_in_dy_and_bf16_equals_fp32_of_same_values():
    p = _layer(12, 8, 4, 8, seed=8, dtype=torch.bfloat16)
    dy = np.random.default_rng(2).standard_normal((12, 8))
    kw = dict(k=2, tau=0.9, renormalize=True, cap_num=5, cap_den=4)
    a = _grads(p, dy, **kw)
    b = _grads(p, 2.0 * dy, **kw)
    pf = {n: (v.float() if v.dtype == torch.bfloat16 else v) for n, v in p.items()}
    c = _grads(pf, dy, **kw)
    for _, gname in NAMES:
        np.testing.assert_array_equal(b[gname], 2.0 * a[gname])
        np.testing.assert_array_equal(c[gname], a[gname])


def test_token_subset_and_single_entries_match_the_full_backward():
    # the per-token mode (dx, dgate of listed tokens) and the single-entry
    # weight gradients, used where the full backward is too large, agree with
    # the finite-difference-pinned full backward
    T, d, E, d_ff = 24, 8, 4, 6
    p = _layer(T, d, E, d_ff, seed=21)
    dy = torch.randn((T, d), generator=torch.Generator().manual_seed(3)).double().numpy()
    kw = dict(k=2, tau=0.8, renormalize=True, cap_num=3, cap_den=4)
    full = orc.backward(p["x"], p["w_router"], p["bias"], p["w_gate"], p["w_up"], p["w_down"],
                        dy, **kw)
    assert (full["row_of"] < 0).any()
    toks = [0, 5, 6, 17, 23]
    sub = orc.backward(p["x"], p["w_router"], p["bias"], p["w_gate"], p["w_up"], p["w_down"],
                       dy, tokens=toks, **kw)
    np.testing.assert_allclose(sub["dx"], full["dx"][toks], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(sub["dgate"], full["dgate"][toks], rtol=1e-13, atol=1e-15)
    rng = np.random.default_rng(0)
    ents = []
    for name, shape in (("dw_gate", (E, d, d_ff)), ("dw_up", (E, d, d_ff)),
                        ("dw_down", (E, d_ff, d))):
        for _ in range(12):
            ents.append((name,) + tuple(int(rng.integers(0, s)) for s in shape))
    got = orc.backward_weight_entries(p["x"], p["w_gate"], p["w_up"], p["w_down"], dy,
                                      full["idx"], full["gate"], full["row_of"], ents)
    want = np.array([full[n][e, a, b] for n, e, a, b in ents])
    scale = max(np.abs(full[n]).max() for n in ("dw_gate", "dw_up", "dw_down"))
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-13 * scale)


def _counts(idx):
    return (np.asarray(idx) >= 0).sum(axis=1)


@pytest.mark.parametrize("renorm,cap", [(True, (0, 0)), (False, (0, 0)), (True, (3, 4))])
def test_dynamic_count_gradients_match_finite_differences(renorm, cap):
    # each token takes 1..3 of 4 experts (the fewest whose softmax mass reaches
    # 0.8); the count is piecewise constant in the logits like the top-k choice,
    # and the gates renormalise over the experts actually taken
    T, d, E, d_ff = 9, 5, 4, 4
    p = _layer(T, d, E, d_ff, seed=40 + int(renorm) + cap[0])
    dy = torch.randn((T, d), generator=torch.Generator().manual_seed(41)).double().numpy()
    kw = dict(k=3, tau=1.5, renormalize=renorm, cap_num=cap[0], cap_den=cap[1], k_min=1,
              threshold=0.8)
    got = _fd_check(p, dy, kw)
    n = _counts(got["idx"])
    assert n.min() < n.max(), n          # the counts really vary
    if cap == (3, 4):
        assert (got["row_of"] < 0).any() and (got["idx"] >= 0).sum() > (got["row_of"] >= 0).sum()


def test_dynamic_count_limits_reduce_to_fixed_top_k():
    # threshold above 1 (never reached): every token takes k experts, the
    # capacity from the realised k T assignments is the fixed one, and the
    # gradients are those of the fixed-k routing, bit for bit; k_min = k with a
    # small threshold gives the same
    T, d, E, d_ff = 16, 6, 5, 6
    p = _layer(T, d, E, d_ff, seed=44)
    dy = np.random.default_rng(4).standard_normal((T, d))
    base = dict(k=3, tau=0.9, renormalize=True, cap_num=5, cap_den=4)
    want = _grads(p, dy, **base)
    for kmin, th in ((1, 1.5), (3, 1e-3)):
        got = _grads(p, dy, k_min=kmin, threshold=th, **base)
        np.testing.assert_array_equal(got["idx"], want["idx"])
        for _, gname in NAMES + [(None, "dgate")]:
            np.testing.assert_array_equal(got[gname], want[gname])
    # k_min = 1 with a threshold below every top probability: top-1 routing
    t1 = _grads(p, dy, **dict(base, k=1))
    g1 = _grads(p, dy, k_min=1, threshold=1e-6, **base)
    assert (_counts(g1["idx"]) == 1).all()
    for _, gname in NAMES:
        np.testing.assert_allclose(g1[gname], t1[gname], rtol=0,
                                   atol=1e-12 * (np.abs(t1[gname]).max() + 1e-300))


def test_dynamic_router_backward_alone_matches_the_full_backward():
    # dlogit from the gate gradients alone, summed over tokens, is the full
    # backward's dbias; x^T dlogit its router weight gradient
    T, d, E, d_ff = 30, 8, 6, 8
    p = _layer(T, d, E, d_ff, seed=46)
    dy = np.random.default_rng(5).standard_normal((T, d))
    kw = dict(k=4, tau=0.7, renormalize=True, cap_num=0, cap_den=0, k_min=2, threshold=0.8)
    g = _grads(p, dy, **kw)
    n = _counts(g["idx"])
    assert n.min() == 2 and n.max() > 2
    dl = orc.router_backward(g["logits"], g["idx"], g["gate"], g["dgate"], 0.7, True)
    np.testing.assert_allclose(dl.sum(axis=0), g["dbias"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(p["x"].double().numpy().T @ dl, g["dw_router"], rtol=1e-11,
                               atol=1e-13)
    assert (g["dgate"][g["idx"] < 0] == 0).all()

"""Pins of the oracle's dynamic expert count (each token takes k_min .. k
experts: the fewest whose softmax mass reaches a threshold; the TorchTitan
1K-GPU article, section 2.1, has each token activate 2-4 experts) and of the
capacity taken from the realised number of assignments.

Expected values come from a hand-worked example (softmax probabilities
0.4 / 0.3 / 0.2 / 0.1 by construction), an exact tie, the limits that reduce
to the static top-k routing (threshold below every mass: k_min experts;
above 1: k experts), brute-force keep decisions and a dense-mixture
evaluation of the whole layer -- never from the oracle itself."""
import math

import numpy as np
import pytest
import torch
from scipy.special import erf

from oracle import oracle as orc

LN = [math.log(0.4), math.log(0.3), math.log(0.2), math.log(0.1)]


def _route(lg, k, kmin, th, tau=1.0, renorm=True):
    return orc.route(np.asarray(lg, dtype=np.float64)[None, :], k, tau, renorm, kmin, th)


@pytest.mark.parametrize("th,kt", [(0.35, 1), (0.65, 2), (0.85, 3), (0.95, 4)])
def test_hand_worked_cumulative_mass(th, kt):
    # p = 0.4, 0.3, 0.2, 0.1 exactly (up to rounding); cumulative 0.4, 0.7, 0.9, 1.0
    idx, gate = _route(LN, 4, 1, th)
    want_idx = [0, 1, 2, 3][:kt] + [-1] * (4 - kt)
    assert idx[0].tolist() == want_idx
    mass = sum([0.4, 0.3, 0.2, 0.1][:kt])
    want = [v / mass for v in [0.4, 0.3, 0.2, 0.1][:kt]] + [0.0] * (4 - kt)
    np.testing.assert_allclose(gate[0], want, rtol=1e-14, atol=0)
    # raw gates: the probabilities themselves
    _, raw = _route(LN, 4, 1, th, renorm=False)
    np.testing.assert_allclose(raw[0], [0.4, 0.3, 0.2, 0.1][:kt] + [0.0] * (4 - kt), rtol=1e-14)


def test_floor_cap_temperature_and_expert_order():
    # k_min is a floor, k a cap
    idx, _ = _route(LN, 4, 2, 0.35)
    assert idx[0].tolist() == [0, 1, -1, -1]
    idx, _ = _route(LN, 3, 1, 0.95)
    assert idx[0].tolist() == [0, 1, 2]
    # tau = 0.5 squares the probabilities: 0.16, 0.09, 0.04, 0.01 over 0.30,
    # cumulative 0.533, 0.833, 0.967; experts stored in another order
    perm = [2, 0, 3, 1]                      # expert e holds LN[perm[e]]
    lg = [LN[perm[e]] for e in range(4)]     # ranks: expert 1 (0.4), 3 (0.3), 0 (0.2), 2 (0.1)
    idx, gate = _route(lg, 4, 1, 0.8, tau=0.5)
    assert idx[0].tolist() == [1, 3, -1, -1]
    np.testing.assert_allclose(gate[0, :2], [0.16 / 0.25, 0.09 / 0.25], rtol=1e-13)
    idx, _ = _route(lg, 4, 1, 0.9, tau=0.5)
    assert idx[0].tolist() == [1, 3, 0, -1]


def test_mass_exactly_at_the_threshold_stops_there():
    # two equal logits: p = 0.5 each, exactly; a threshold of 0.5 is reached by one
    idx, gate = _route([0.25, 0.25], 2, 1, 0.5)
    assert idx[0].tolist() == [0, -1] and gate[0].tolist() == [1.0, 0.0]


@pytest.mark.parametrize("renorm", [True, False])
def test_limits_reduce_to_static_top_k(renorm):
    rng = np.random.default_rng(3)
    lg = rng.normal(size=(200, 9))
    for kmin, k in ((1, 4), (2, 4), (3, 5)):
        lo_i, lo_g = orc.route(lg, k, 0.7, renorm, kmin, 1e-300)
        st_i, st_g = orc.route(lg, kmin, 0.7, renorm)
        assert (lo_i[:, :kmin] == st_i).all() and (lo_i[:, kmin:] == -1).all()
        np.testing.assert_allclose(lo_g[:, :kmin], st_g, rtol=1e-14)
        assert (lo_g[:, kmin:] == 0).all()
        hi_i, hi_g = orc.route(lg, k, 0.7, renorm, kmin, 2.0)
        st_i, st_g = orc.route(lg, k, 0.7, renorm)
        assert (hi_i == st_i).all()
        np.testing.assert_allclose(hi_g, st_g, rtol=1e-14)


def test_count_is_monotone_in_the_threshold_and_minimal():
    rng = np.random.default_rng(4)
    lg = rng.normal(size=(300, 12)) * 2
    prev = None
    for th in (0.2, 0.4, 0.6, 0.8, 0.9, 0.99):
        idx, gate = orc.route(lg, 4, 0.5, True, 2, th)
        kt = (idx >= 0).sum(1)
        assert ((kt >= 2) & (kt <= 4)).all()
        if prev is not None:
            assert (kt >= prev).all()
        prev = kt
        np.testing.assert_allclose(gate.sum(1), 1.0, rtol=1e-13)
        # the chosen experts are the kt best of the static ranking
        st, _ = orc.route(lg, 4, 0.5, True)
        for t in range(lg.shape[0]):
            assert idx[t, :kt[t]].tolist() == st[t, :kt[t]].tolist()


def _brute_keep(idx, C):
    """keep[t][j] iff idx[t][j] >= 0 and fewer than C earlier tokens chose it."""
    T, k = idx.shape
    keep = np.zeros((T, k), dtype=bool)
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            if e < 0:
                continue
            keep[t, j] = sum(1 for tp in range(t) if e in idx[tp]) < C
    return keep


def test_realised_capacity_and_dispatch_skip_empty_slots():
    rng = np.random.default_rng(5)
    lg = rng.normal(size=(80, 6))
    idx, _ = orc.route(lg, 4, 0.6, True, 2, 0.7)
    A = int((idx >= 0).sum())
    assert 2 * 80 <= A < 4 * 80
    C = orc.capacity_realised(idx, 6, 5, 4)
    assert C == -(-5 * A // (4 * 6))            # ceil(1.25 A / E)
    assert orc.capacity_realised(idx, 6, 0, 0) == 80   # no limit: C = T
    d = orc.dispatch(idx, 6, C)
    keep = _brute_keep(idx, C)
    assert ((d["row_of"] >= 0) == keep).all()
    assert d["count"].sum() == A
    assert (d["pos"][idx < 0] == -1).all()


def _ffn(x, wg, wu, wd):
    g = x @ wg
    u = x @ wu
    return (0.5 * g * (1.0 + erf(g / np.sqrt(2.0))) * u) @ wd


def test_whole_layer_matches_dense_mixture_with_dynamic_counts():
    T, d, E, F = 60, 16, 5, 24
    gen = torch.Generator().manual_seed(6)
    r = lambda *s, sc=1.0: torch.randn(*s, generator=gen) * sc
    x, wr = r(T, d), r(d, E, sc=0.5)
    wg, wu, wd = r(E, d, F, sc=0.3), r(E, d, F, sc=0.3), r(E, F, d, sc=0.3)
    out = orc.forward(x, wr, None, wg, wu, wd, k=4, tau=0.5, renormalize=True, cap_num=1,
                      cap_den=1, k_min=2, threshold=0.8)
    idx, gate = out["idx"], out["gate"]
    C = orc.capacity_realised(idx, E, 1, 1)
    keep = _brute_keep(idx, C)
    assert keep.sum() < (idx >= 0).sum()          # some drops at capacity factor 1
    x64 = x.double().numpy()
    dense = np.stack([_ffn(x64, wg[e].double().numpy(), wu[e].double().numpy(),
                           wd[e].double().numpy()) for e in range(E)])      # [E, T, d]
    want = np.zeros((T, d))
    for t in range(T):
        for j in range(4):
            if keep[t, j]:
                want[t] += gate[t, j] * dense[idx[t, j], t]
    np.testing.assert_allclose(out["y"], want, rtol=1e-10, atol=1e-12)

"""Pins of the fp64 oracle to things other than itself.

Every expected value here comes from an independent route: numpy/scipy library
routines (matmul, stable argsort, lexsort, softmax, expit, erf), brute-force
enumeration on tiny inputs, closed forms, or a textbook table
(tests/golden/normal_cdf.txt).  None of them calls the oracle to make its
expectation.  The cases are chosen so that a plausible slip in the oracle -- a
dropped bias, a transposed weight, a wrong tie-break, temperature applied the
wrong way, choice-major instead of token-order drops, tanh-GELU instead of erf,
a missing renormalisation -- fails at least one of them.
"""
import itertools
import os

import numpy as np
import pytest
import torch
from scipy.special import erf, expit, softmax

from oracle import oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, scale=1.0, dtype=torch.float32):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(dtype)


def _f64(t):
    return t.double().numpy()


def _ffn_dense(x, wg, wu, wd):
    """GeGLU FFN of every token through one expert, numpy + scipy erf."""
    g = x @ wg
    u = x @ wu
    h = 0.5 * g * (1.0 + erf(g / np.sqrt(2.0))) * u
    return h @ wd


def _brute_topk(l, k):
    """Best k-subset by sum of logits, ties -> lexicographically first index
    tuple; then ordered by (logit desc, index asc).  Integer logits only."""
    E = len(l)
    best, best_s = None, None
    for S in itertools.combinations(range(E), k):
        s = sum(l[e] for e in S)
        if best is None or s > best_s:
            best, best_s = S, s
    return sorted(best, key=lambda e: (-l[e], e))


def _brute_keep(idx, C):
    """keep[t][j] iff fewer than C earlier tokens chose the same expert."""
    T, k = idx.shape
    keep = np.zeros((T, k), dtype=bool)
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            earlier = sum(1 for tp in range(t) if e in idx[tp])
            keep[t, j] = earlier < C
    return keep


def _random_choices(T, E, k, seed):
    rng = np.random.default_rng(seed)
    return np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)


# ---------------------------------------------------------------- logits

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_logits_match_numpy_matmul_with_bias(dtype):
    T, d, E = 37, 24, 5
    x = _rand((T, d), 1, dtype=dtype)
    wr = _rand((d, E), 2, 0.2, dtype=dtype)
    b = _rand((E,), 3)
    got = orc.logits(x, wr, b)
    want = _f64(x) @ _f64(wr) + _f64(b)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    got0 = orc.logits(x, wr, None)
    np.testing.assert_allclose(got0, _f64(x) @ _f64(wr), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- top-k

@pytest.mark.parametrize("E", [1, 2, 3, 5, 6])
def test_topk_matches_bruteforce_with_ties(E):
    rng = np.random.default_rng(E)
    T = 150
    l = rng.integers(-2, 3, size=(T, E)).astype(np.float64)   # many exact ties
    for k in range(1, E + 1):
        idx, _ = orc.route(l, k, 1.0, True)
        for t in range(T):
            assert list(idx[t]) == _brute_topk(list(l[t]), k), (t, l[t], k)
        np.testing.assert_array_equal(idx, np.argsort(-l, axis=1, kind="stable")[:, :k])


def test_topk_real_valued_and_signed_zero():
    l = _f64(_rand((300, 17), 11))
    idx, _ = orc.route(l, 4, 0.3, True)
    np.testing.assert_array_equal(idx, np.argsort(-l, axis=1, kind="stable")[:, :4])
    # -0.0 and +0.0 compare equal: the lower index wins
    z = np.array([[-0.0, 0.0, -1.0], [0.0, -0.0, -1.0]])
    idx, _ = orc.route(z, 1, 1.0, False)
    assert idx[:, 0].tolist() == [0, 0]


# ---------------------------------------------------------------- gates

@pytest.mark.parametrize("tau", [0.3, 1.0, 2.5])
def test_gates_closed_forms(tau):
    l = _f64(_rand((64, 2), 5, 2.0))
    # E = 2, top-1, raw probability: p_max = sigmoid(|l0 - l1| / tau)
    idx, g = orc.route(l, 1, tau, False)
    np.testing.assert_allclose(g[:, 0], expit(np.abs(l[:, 0] - l[:, 1]) / tau), rtol=1e-14)
    # E = 2, top-2 renormalised: sigmoid of the ordered gap
    idx, g = orc.route(l, 2, tau, True)
    gap = l[np.arange(64), idx[:, 0]] - l[np.arange(64), idx[:, 1]]
    np.testing.assert_allclose(g[:, 0], expit(gap / tau), rtol=1e-14)
    np.testing.assert_allclose(g[:, 1], expit(-gap / tau), rtol=1e-13)
    # k = E renormalised == softmax(l / tau) in rank order
    l6 = _f64(_rand((40, 6), 6, 1.5))
    idx, g = orc.route(l6, 6, tau, True)
    p = softmax(l6 / tau, axis=1)
    np.testing.assert_allclose(g, np.take_along_axis(p, idx, axis=1), rtol=1e-13)
    # k < E raw: gate = softmax probability of the chosen expert (not renormalised)
    idx, g = orc.route(l6, 2, tau, False)
    np.testing.assert_allclose(g, np.take_along_axis(p, idx, axis=1), rtol=1e-13)
    # k < E renormalised: divided by the chosen mass
    idx, g = orc.route(l6, 2, tau, True)
    pc = np.take_along_axis(p, idx, axis=1)
    np.testing.assert_allclose(g, pc / pc.sum(1, keepdims=True), rtol=1e-13)
    np.testing.assert_allclose(g.sum(1), 1.0, rtol=1e-14)
    assert np.all(g[:, 0] >= g[:, 1])


def test_gates_shift_invariant_and_topk_temperature_free():
    l = _f64(_rand((50, 8), 7))
    i1, g1 = orc.route(l, 3, 0.3, True)
    i2, g2 = orc.route(l + 123.25, 3, 0.3, True)
    i3, _ = orc.route(l, 3, 7.0, True)
    np.testing.assert_array_equal(i1, i2)
    np.testing.assert_array_equal(i1, i3)
    np.testing.assert_allclose(g1, g2, rtol=1e-10)


# ---------------------------------------------------------------- capacity

def test_capacity_values():
    # exact integers at the measured workloads
    assert orc.capacity(16384, 128, 2, 5, 4) == 320
    assert orc.capacity(32768, 64, 2, 5, 4) == 1280
    assert orc.capacity(65536, 8, 2, 5, 4) == 20480
    # ceiling, not floor: 1.25 * 1 * 10 / 3 = 4.1667 -> 5
    assert orc.capacity(10, 3, 1, 5, 4) == 5
    assert orc.capacity(12, 3, 1, 1, 1) == 4
    # no limit -> T; zero factor -> 0
    assert orc.capacity(777, 5, 2, 0, 0) == 777
    assert orc.capacity(777, 5, 2, 0, 1) == 0


# ---------------------------------------------------------------- dispatch

@pytest.mark.parametrize("C", [0, 1, 3, 7, 40])
@pytest.mark.parametrize("E,k", [(5, 2), (4, 1), (6, 3), (3, 3)])
def test_dispatch_matches_bruteforce(C, E, k):
    T = 40
    idx = _random_choices(T, E, k, seed=C * 31 + E * 7 + k)
    got = orc.dispatch(idx, E, C)
    keep = _brute_keep(idx, C)
    count = np.bincount(idx.reshape(-1), minlength=E)
    np.testing.assert_array_equal(got["count"], count)
    kept = np.bincount(idx[keep], minlength=E)
    np.testing.assert_array_equal(got["kept"], kept)
    np.testing.assert_array_equal(got["kept"], np.minimum(count, C))
    np.testing.assert_array_equal(got["offset"], np.concatenate([[0], np.cumsum(kept)]))
    # permutation: kept assignments sorted by (expert, token) -- numpy lexsort
    tt, jj = np.nonzero(keep)
    order = np.lexsort((tt, idx[tt, jj]))
    np.testing.assert_array_equal(got["token_of_row"], tt[order])
    row_of = np.full((T, k), -1)
    row_of[tt[order], jj[order]] = np.arange(order.size)
    np.testing.assert_array_equal(got["row_of"], row_of)
    assert got["n_kept"] == T * k - int((~keep).sum())


def test_drops_follow_token_order_not_choice_rank():
    # expert 0 is token 0's second choice and token 1's first choice; with
    # C = 1 token order keeps token 0's assignment (a choice-major priority
    # would keep token 1's instead)
    idx = np.array([[1, 0], [0, 2]], dtype=np.int32)
    got = orc.dispatch(idx, 3, 1)
    assert got["row_of"].tolist() == [[1, 0], [-1, 2]]
    assert got["token_of_row"].tolist() == [0, 0, 1]
    assert got["kept"].tolist() == [1, 1, 1] and got["count"].tolist() == [2, 1, 1]


def _brute_keep_choice_order(idx, C):
    """keep[t][j] iff fewer than C assignments to the same expert come before
    (t, j) when all first choices (in token order) precede all second choices."""
    T, k = idx.shape
    keep = np.zeros((T, k), dtype=bool)
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            earlier = sum(1 for jp in range(k) for tp in range(T)
                          if (jp, tp) < (j, t) and idx[tp, jp] == e)
            keep[t, j] = earlier < C
    return keep


@pytest.mark.parametrize("C", [0, 1, 3, 7, 40])
@pytest.mark.parametrize("E,k", [(5, 2), (4, 1), (6, 3), (3, 3)])
def test_choice_order_dispatch_matches_bruteforce(C, E, k):
    T = 40
    idx = _random_choices(T, E, k, seed=C * 37 + E * 11 + k)
    got = orc.dispatch(idx, E, C, policy=1)
    keep = _brute_keep_choice_order(idx, C)
    count = np.bincount(idx.reshape(-1), minlength=E)
    np.testing.assert_array_equal(got["count"], count)
    kept = np.bincount(idx[keep], minlength=E)
    np.testing.assert_array_equal(got["kept"], kept)
    np.testing.assert_array_equal(got["offset"], np.concatenate([[0], np.cumsum(kept)]))
    # rows of an expert in priority order: (expert, choice rank, token) -- lexsort
    tt, jj = np.nonzero(keep)
    order = np.lexsort((tt, jj, idx[tt, jj]))
    np.testing.assert_array_equal(got["token_of_row"], tt[order])
    row_of = np.full((T, k), -1)
    row_of[tt[order], jj[order]] = np.arange(order.size)
    np.testing.assert_array_equal(got["row_of"], row_of)


def test_choice_order_differs_from_token_order():
    # worked by hand: expert 1 is token 0's second choice and token 1's first;
    # with C = 1 token order keeps token 0's, choice order keeps token 1's
    idx = np.array([[0, 1], [1, 0], [0, 1]], dtype=np.int32)
    tok = orc.dispatch(idx, 2, 1, policy=0)
    cho = orc.dispatch(idx, 2, 1, policy=1)
    assert tok["row_of"].tolist() == [[0, 1], [-1, -1], [-1, -1]]
    assert cho["row_of"].tolist() == [[0, -1], [1, -1], [-1, -1]]
    assert tok["token_of_row"].tolist() == [0, 0] and cho["token_of_row"].tolist() == [0, 1]
    # k = 1: the two orders coincide
    one = np.array([[2], [0], [2], [1], [2]], dtype=np.int32)
    for C in (0, 1, 2):
        a, b = orc.dispatch(one, 3, C, 0), orc.dispatch(one, 3, C, 1)
        assert a["row_of"].tolist() == b["row_of"].tolist()


# ---------------------------------------------------------------- load telemetry

def test_load_stats_closed_forms():
    E = 8
    # uniform load: every ratio at its floor
    s = orc.load_stats(np.full(E, 5, np.int32), C=5)
    assert s.tolist() == [5.0, 5.0, 5.0, 1.0, 0.0, 0.0, 0.0, 0.0]
    # everything on one expert: max/mean = E, deviation E - 1, CV = sqrt(E - 1)
    one = np.zeros(E, np.int32)
    one[3] = 64
    s = orc.load_stats(one, C=10)
    assert s[0] == 8.0 and s[1] == 64.0 and s[2] == 0.0 and s[3] == E
    assert s[4] == E - 1 and abs(s[5] - np.sqrt(E - 1)) < 1e-15
    assert s[6] == 64 - 10 and s[7] == E - 1
    # worked by hand: counts 3, 1, 0, 4 (mean 2), C = 2
    s = orc.load_stats(np.array([3, 1, 0, 4], np.int32), C=2)
    assert s[:5].tolist() == [2.0, 4.0, 0.0, 2.0, 1.0]
    assert abs(s[5] - np.sqrt(10.0 / 4.0) / 2.0) < 1e-15
    assert s[6] == 3.0 and s[7] == 1.0
    # no assignments at all: ratios 0, every expert empty
    assert orc.load_stats(np.zeros(4, np.int32), C=0).tolist() == [0.0] * 7 + [4.0]


def test_load_stats_deviation_is_largest_either_side():
    # the largest deviation may sit below the mean: counts 10, 10, 10, 2
    s = orc.load_stats(np.array([10, 10, 10, 2], np.int32), C=100)
    assert s[0] == 8.0 and s[4] == 6.0 / 8.0 and s[3] == 10.0 / 8.0


# ---------------------------------------------------------------- MLP router (variant)

def _gelu(v):
    return 0.5 * v * (1.0 + erf(v / np.sqrt(2.0)))


def _mlp_shapes(T=6, d=64, r=16, m=24, E=5):
    z = lambda *sh: torch.zeros(sh)
    return T, d, r, m, E, z


def test_mlp_router_zero_hidden_weights_give_output_biases():
    T, d, r, m, E, z = _mlp_shapes()
    x = _rand((T, d), 1)
    b3 = _rand((E,), 2)
    pid = _rand((E,), 3)
    out = orc.mlp_router(x, _rand((T, r), 4), 0.7, 1e-6, _rand((d, r), 5), _rand((r,), 6),
                         z(r, m), None, z(m, m), None, _rand((m, E), 7), b3, pid)
    want = (b3.double() + pid.double()).numpy()    # GELU(0) = 0 ends every path before W3
    np.testing.assert_array_equal(out["logits"], np.tile(want, (T, 1)))


def test_mlp_router_single_path_chain():
    # one nonzero weight per matrix: x[i0] -> u[j0] -> h1[n0] -> h2[n1] -> l[e0];
    # non-square widths so that any transposed index lands elsewhere
    T, d, r, m, E, z = _mlp_shapes()
    i0, j0, n0, n1, e0 = 5, 3, 7, 11, 2
    a, b, c, w = (float(np.float32(v)) for v in (0.8, 1.3, -0.9, 2.1))   # as stored (fp32)
    x = _rand((T, d), 11)
    wd, w1, w2, w3 = z(d, r), z(r, m), z(m, m), z(m, E)
    wd[i0, j0], w1[j0, n0], w2[n0, n1], w3[n1, e0] = a, b, c, w
    out = orc.mlp_router(x, None, 0.0, 1e-3, wd, None, w1, None, w2, None, w3, None, None,
                         want_hidden=True)
    v = a * x[:, i0].double().numpy()
    zz = v / np.sqrt(v * v / r + 1e-3)
    want = np.zeros((T, E))
    want[:, e0] = w * _gelu(c * _gelu(b * zz))
    np.testing.assert_allclose(out["logits"], want, rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(out["z"][:, j0], zz, rtol=1e-15)
    assert (np.delete(out["z"], j0, axis=1) == 0).all()


def test_mlp_router_rms_norm_closed_form_and_depth_average():
    # u = 0.5 on every coordinate plus gamma * prev: z = v / sqrt(mean v^2 + eps)
    T, d, r, m, E, z = _mlp_shapes(T=3, d=64, r=4, m=8, E=3)
    x = torch.zeros((T, d))
    x[:, 0] = 1.0
    wd = torch.zeros((d, r))
    wd[0, :] = 0.5
    prev = torch.tensor([[1.0, -1.0, 2.0, 0.0], [0.0, 0.0, 0.0, 0.0], [4.0, 4.0, 4.0, 4.0]])
    gamma, eps = 0.25, 0.0625
    out = orc.mlp_router(x, prev, gamma, eps, wd, None, z(r, m), None, z(m, m), None,
                         z(m, E), None, None, want_hidden=True)
    v = 0.5 + gamma * prev.double().numpy()
    want = v / np.sqrt((v * v).mean(1, keepdims=True) + eps)
    np.testing.assert_allclose(out["z"], want, rtol=1e-15)
    # row 1: v = 0.5 everywhere -> z = 0.5 / sqrt(0.25 + 0.0625) = 0.894427...
    assert abs(out["z"][1, 0] - 0.5 / np.sqrt(0.3125)) < 1e-15


def test_mlp_router_scale_invariance_without_eps():
    T, d, r, m, E, z = _mlp_shapes()
    x, prev = _rand((T, d), 21), _rand((T, r), 22)
    ws = [_rand((d, r), 23, d ** -0.5), _rand((r,), 24), _rand((r, m), 25, r ** -0.5),
          _rand((m,), 26), _rand((m, m), 27, m ** -0.5), _rand((m,), 28),
          _rand((m, E), 29, m ** -0.5), _rand((E,), 30)]
    a = orc.mlp_router(x, prev, 0.6, 0.0, ws[0], ws[1], *ws[2:], None)["logits"]
    # scaling x, bd and prev by 4 (exact in fp32) scales v by 4; the norm removes it
    b = orc.mlp_router(x * 4, prev * 4, 0.6, 0.0, ws[0], ws[1] * 4, *ws[2:], None)["logits"]
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


def test_mlp_router_identity_layers_and_biases():
    # W1 = [I | 0] (r < m) and W2 = I: h1 = GELU(z + b1) on the first r units, GELU(b1) on
    # the rest; h2 = GELU(h1 + b2)
    T, d, r, m, E, z = _mlp_shapes(T=4, d=64, r=8, m=12, E=3)
    x = _rand((T, d), 31)
    w1 = z(r, m)
    w1[:, :r] = torch.eye(r)
    b1, b2 = _rand((m,), 32), _rand((m,), 33)
    out = orc.mlp_router(x, None, 0.0, 1e-6, _rand((d, r), 34, d ** -0.5), None, w1, b1,
                         torch.eye(m), b2, _rand((m, E), 35), None, None, want_hidden=True)
    zz = out["z"]
    pre1 = np.concatenate([zz, np.zeros((T, m - r))], 1) + b1.double().numpy()
    np.testing.assert_allclose(out["h1"], _gelu(pre1), rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(out["h2"], _gelu(out["h1"] + b2.double().numpy()), rtol=1e-14,
                               atol=1e-300)


def test_mlp_router_expert_permutation():
    T, d, r, m, E, z = _mlp_shapes()
    args = [_rand((T, d), 41), _rand((T, r), 42), 0.3, 1e-6, _rand((d, r), 43), _rand((r,), 44),
            _rand((r, m), 45), _rand((m,), 46), _rand((m, m), 47), _rand((m,), 48)]
    w3, b3, pid = _rand((m, E), 49), _rand((E,), 50), _rand((E,), 51)
    perm = np.array([3, 0, 4, 1, 2])
    a = orc.mlp_router(*args, w3, b3, pid)["logits"]
    b = orc.mlp_router(*args, w3[:, perm].contiguous(), b3[perm], pid[perm])["logits"]
    np.testing.assert_array_equal(a[:, perm], b)


# ---------------------------------------------------------------- expert FFN

def test_gelu_is_erf_form_against_normal_table():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "normal_cdf.txt"))
            if l.strip() and not l.startswith("#")]
    v = np.array([float(r[0]) for r in rows], dtype=np.float32)
    phi = np.array([float(r[1]) for r in rows])
    one = np.ones((1, 1, 1), dtype=np.float32)
    # d = d_ff = 1 and unit weights: o = GELU(v) * v = v^2 * Phi(v)
    o = orc.ffn_rows(np.arange(len(v)), np.zeros(len(v), np.int32), v.reshape(-1, 1),
                     one, one, one)
    np.testing.assert_allclose(o[:, 0], v.astype(np.float64) ** 2 * phi, rtol=1e-15, atol=1e-300)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_single_expert_layer_is_dense_geglu_ffn(dtype):
    T, d, F = 20, 16, 24
    x = _rand((T, d), 21, dtype=dtype)
    wr = _rand((d, 1), 22, dtype=dtype)
    wg = _rand((1, d, F), 23, 0.25, dtype)
    wu = _rand((1, d, F), 24, 0.25, dtype)
    wd = _rand((1, F, d), 25, 0.2, dtype)
    out = orc.forward(x, wr, None, wg, wu, wd, k=1, tau=1.0, renormalize=False,
                      cap_num=0, cap_den=0)
    assert np.all(out["gate"] == 1.0)
    want = _ffn_dense(_f64(x), _f64(wg[0]), _f64(wu[0]), _f64(wd[0]))
    np.testing.assert_allclose(out["y"], want, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- whole layer

def _dense_mixture(x, wr, b, wg, wu, wd, k, tau, renorm, C):
    """Every expert on every token, masked by brute-force routing and drops."""
    X = _f64(x)
    L = X @ _f64(wr) + (0 if b is None else _f64(b))
    T, E = L.shape
    idx = np.argsort(-L, axis=1, kind="stable")[:, :k]
    p = softmax(L / tau, axis=1)
    pc = np.take_along_axis(p, idx, axis=1)
    g = pc / pc.sum(1, keepdims=True) if renorm else pc
    keep = _brute_keep(idx, C)
    y = np.zeros_like(X)
    for e in range(E):
        fe = _ffn_dense(X, _f64(wg[e]), _f64(wu[e]), _f64(wd[e]))
        m = ((idx == e) & keep) * g
        y += m.sum(1, keepdims=True) * fe
    return y


@pytest.mark.parametrize("renorm", [False, True])
@pytest.mark.parametrize("cap", [(0, 0), (5, 4), (1, 2), (0, 1)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_layer_matches_dense_mixture_bruteforce(renorm, cap, dtype):
    T, d, E, k, F, tau = 12, 8, 5, 3, 6, 0.7
    x = _rand((T, d), 31, dtype=dtype)
    wr = _rand((d, E), 32, 0.5, dtype)
    b = _rand((E,), 33, 0.3)
    wg = _rand((E, d, F), 34, 0.35, dtype)
    wu = _rand((E, d, F), 35, 0.35, dtype)
    wd = _rand((E, F, d), 36, 0.4, dtype)
    C = orc.capacity(T, E, k, *cap)
    out = orc.forward(x, wr, b, wg, wu, wd, k=k, tau=tau, renormalize=renorm,
                      cap_num=cap[0], cap_den=cap[1])
    want = _dense_mixture(x, wr, b, wg, wu, wd, k, tau, renorm, C)
    np.testing.assert_allclose(out["y"], want, rtol=1e-11, atol=1e-12)
    if cap == (0, 1):
        assert np.all(out["y"] == 0.0) and out["n_kept"] == 0


def test_all_experts_renormalised_is_softmax_mixture():
    T, d, E, F, tau = 9, 8, 4, 8, 0.45
    x = _rand((T, d), 41)
    wr = _rand((d, E), 42, 0.6)
    wg = _rand((E, d, F), 43, 0.3)
    wu = _rand((E, d, F), 44, 0.3)
    wd = _rand((E, F, d), 45, 0.3)
    out = orc.forward(x, wr, None, wg, wu, wd, k=E, tau=tau, renormalize=True,
                      cap_num=0, cap_den=0)
    X = _f64(x)
    p = softmax((X @ _f64(wr)) / tau, axis=1)
    want = sum(p[:, e:e + 1] * _ffn_dense(X, _f64(wg[e]), _f64(wu[e]), _f64(wd[e]))
               for e in range(E))
    np.testing.assert_allclose(out["y"], want, rtol=1e-12, atol=1e-13)


def test_token_sample_and_logits_override_agree_with_full_forward():
    T, d, E, k, F = 64, 16, 6, 2, 12
    x = _rand((T, d), 51, dtype=torch.bfloat16)
    wr = _rand((d, E), 52, 0.25, torch.bfloat16)
    wg = _rand((E, d, F), 53, 0.25, torch.bfloat16)
    wu = _rand((E, d, F), 54, 0.25, torch.bfloat16)
    wd = _rand((E, F, d), 55, 0.25, torch.bfloat16)
    kw = dict(k=k, tau=0.3, renormalize=True, cap_num=5, cap_den=4)
    full = orc.forward(x, wr, None, wg, wu, wd, **kw)
    toks = [0, 5, 17, 63]
    part = orc.forward(x, wr, None, wg, wu, wd, tokens=toks, **kw)
    np.testing.assert_array_equal(part["y"], full["y"][toks])
    over = orc.forward(x, wr, None, wg, wu, wd, logits_in=full["logits"], **kw)
    np.testing.assert_array_equal(over["y"], full["y"])


@pytest.mark.parametrize("C", [0, 1, 3, 7, 40])
@pytest.mark.parametrize("policy", [0, 1])
@pytest.mark.parametrize("E,k", [(5, 2), (4, 1), (6, 3)])
def test_padded_layout_matches_bruteforce(C, policy, E, k):
    # each expert owns rows e*C .. e*C + C - 1; its kept assignments fill the
    # first rows in priority order, the rest are empty (-1)
    T = 40
    idx = _random_choices(T, E, k, seed=C * 29 + E * 7 + k + 100 * policy)
    got = orc.dispatch(idx, E, C, policy=policy, layout=1)
    order = [(t, j) for t in range(T) for j in range(k)] if policy == 0 else \
        [(t, j) for j in range(k) for t in range(T)]
    seen = np.zeros(E, dtype=np.int64)
    row_of = np.full((T, k), -1)
    tor = np.full(E * C, -1)
    for t, j in order:
        e = idx[t, j]
        if seen[e] < C:
            row_of[t, j] = e * C + seen[e]
            tor[e * C + seen[e]] = t
        seen[e] += 1
    np.testing.assert_array_equal(got["row_of"], row_of)
    np.testing.assert_array_equal(got["token_of_row"], tor)
    np.testing.assert_array_equal(got["offset"], np.arange(E + 1) * C)
    assert got["n_rows"] == E * C and got["n_kept"] == int((row_of >= 0).sum())
    # the same assignments are kept as in the compact layout
    compact = orc.dispatch(idx, E, C, policy=policy)
    np.testing.assert_array_equal(compact["row_of"] >= 0, row_of >= 0)
    np.testing.assert_array_equal(got["count"], compact["count"])

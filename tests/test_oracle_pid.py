"""Pins of the oracle's load-balance PID controller (the MLP router's PID
balance control, "AMD MI300X平台上的MoE模型训练实践", section 3.2; the gains
ramped over a warmup, same page's training notes), read as one textbook
discrete PID loop per expert on the relative load error, output = additive
logit bias.

Expected values come from a hand-worked example, the closed forms of a
constant error sequence, linearity in the warmup scale, the zero-sum of the
errors, and a closed-loop property (the controller, fed back through a
router, evens out a skewed load; with any sign wrong it does not)."""
import numpy as np
import pytest

from oracle import oracle as orc


def _zero(E):
    return np.zeros((2, E))


def test_hand_worked_two_steps():
    # counts 10, 30, 20, 20: mean 20, errors +0.5, -0.5, 0, 0
    c = np.array([10, 30, 20, 20])
    st, b = orc.pid_update(c, _zero(4), kp=1.0, ki=0.5, kd=0.25)
    # first step: I = err, D = err - 0: bias = (1 + 0.5 + 0.25) err
    np.testing.assert_array_equal(b, [0.875, -0.875, 0.0, 0.0])
    np.testing.assert_array_equal(st, [[0.5, -0.5, 0, 0], [0.5, -0.5, 0, 0]])
    # second step, same counts: I = 2 err, D = 0: bias = (1 + 1.0) err
    st2, b2 = orc.pid_update(c, st, kp=1.0, ki=0.5, kd=0.25)
    np.testing.assert_array_equal(b2, [1.0, -1.0, 0.0, 0.0])
    np.testing.assert_array_equal(st2, [[1.0, -1.0, 0, 0], [0.5, -0.5, 0, 0]])
    # the state passed in is left as it was
    np.testing.assert_array_equal(st, [[0.5, -0.5, 0, 0], [0.5, -0.5, 0, 0]])


def test_constant_counts_closed_form():
    rng = np.random.default_rng(3)
    E = 37
    c = rng.integers(0, 500, E)
    m = c.sum() / E
    err = (m - c) / m
    kp, ki, kd = 0.7, 0.05, 0.3
    st = _zero(E)
    for n in range(1, 9):
        st, b = orc.pid_update(c, st, kp, ki, kd)
        want = kp * err + ki * n * err + (kd * err if n == 1 else 0.0)
        np.testing.assert_allclose(b, want, rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(st[0], n * err, rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(st[1], err, rtol=0, atol=0)
    # the errors sum to zero over the experts, so the integral does too
    assert abs(st[0].sum()) <= 1e-12 * np.abs(st[0]).sum()


def test_scale_is_linear_and_leaves_the_state_alone():
    rng = np.random.default_rng(4)
    E = 16
    st0 = rng.standard_normal((2, E))
    c = rng.integers(0, 100, E)
    s1, b1 = orc.pid_update(c, st0, 0.4, 0.1, 0.2, scale=1.0)
    for s in (0.0, 0.25, 0.5):
        ss, bs = orc.pid_update(c, st0, 0.4, 0.1, 0.2, scale=s)
        np.testing.assert_array_equal(ss, s1)
        np.testing.assert_allclose(bs, s * b1, rtol=1e-15, atol=0)


def test_no_assignments_gives_zero_error():
    rng = np.random.default_rng(5)
    E = 8
    st0 = rng.standard_normal((2, E))
    st, b = orc.pid_update(np.zeros(E, np.int32), st0, 0.3, 0.2, 0.1)
    np.testing.assert_array_equal(st[0], st0[0])     # integral unchanged
    np.testing.assert_array_equal(st[1], 0.0)        # previous error now 0
    np.testing.assert_allclose(b, 0.2 * st0[0] + 0.1 * (0.0 - st0[1]), rtol=1e-15)
    # one expert: always at the mean
    st, b = orc.pid_update(np.array([42]), _zero(1), 1.0, 1.0, 1.0)
    assert b[0] == 0.0 and (st == 0).all()


def _imbalance(c):
    m = c.mean()
    return float(np.abs(c - m).max() / m)


@pytest.mark.parametrize("E", [8, 64])
def test_closed_loop_evens_out_a_skewed_load(E):
    # a top-1 router on fixed logits with a Zipf-like preference; each step
    # the counts of the biased router feed the controller
    rng = np.random.default_rng(E)
    T = 4096
    logits = rng.standard_normal((T, E)) - 0.8 * np.log1p(np.arange(E))
    counts = lambda b: np.bincount(np.argmax(logits + b, axis=1), minlength=E)
    first = _imbalance(counts(np.zeros(E)))
    assert first > 1.0

    def run(sign):
        b, s = np.zeros(E), _zero(E)
        for step in range(300):
            scale = min(1.0, (step + 1) / 50)          # gains raised over a warmup
            s, b = orc.pid_update(counts(b), s, kp=sign * 0.3, ki=sign * 0.03,
                                  kd=sign * 0.05, scale=scale)
        return b, _imbalance(counts(b))

    bias, last = run(1.0)
    assert last < min(1.0, 0.1 * first), (first, last)
    # the most preferred expert ends with the lowest bias
    assert bias[0] == bias.min()
    # the same loop with the controller's sign reversed makes the skew worse
    _, worse = run(-1.0)
    assert worse > first, (first, worse)

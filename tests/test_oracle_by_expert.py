"""Pins of the by-expert oracle (oracle/by_expert.py: the expert FFN, combine
and backward with numpy's fp64 matrix product as the step for each sum) to
the row-by-row C oracle, which is itself pinned to library routines, brute
force, closed forms and central finite differences (test_oracle_pins.py,
test_oracle_backward.py).  The two share no arithmetic code: agreement to
fp64 rounding on layers with drops, raw and renormalised gates, both drop
priorities, fp32 and bf16 inputs, and experts split over several row blocks
pins the by-expert form.  A plausible slip in it -- a transposed weight,
the tanh GELU, a gate applied twice, a missing drop, GELU' with the wrong
sign -- moves some output by far more than the 1e-10 used here."""
import numpy as np
import pytest
import torch

from oracle import by_expert
from oracle import oracle as orc

REL = 1e-10


def _layer(T, d, E, d_ff, seed, dtype=torch.float32):
    g = torch.Generator().manual_seed(seed)
    r = lambda *s, sc=1.0: (torch.randn(*s, generator=g) * sc).to(dtype)
    return dict(x=r(T, d), w_router=r(d, E, sc=d ** -0.5), bias=r(E, sc=0.5).float(),
                w_gate=r(E, d, d_ff, sc=d ** -0.5), w_up=r(E, d, d_ff, sc=d ** -0.5),
                w_down=r(E, d_ff, d, sc=d_ff ** -0.5))


def _close(got, want):
    scale = np.abs(want).max()
    assert scale > 0
    err = np.abs(got - want).max() / scale
    assert err <= REL, err


CASES = [
    # T, d, E, k, d_ff, tau, renorm, cap, policy, dtype, chunk
    (200, 48, 5, 2, 80, 0.7, True, (5, 4), 0, torch.float32, 16),
    (150, 32, 4, 1, 64, 1.0, False, (0, 0), 0, torch.bfloat16, 7),
    (120, 40, 6, 3, 56, 0.5, False, (3, 4), 1, torch.float32, 1000),
    (90, 32, 3, 2, 32, 0.3, True, (1, 3), 0, torch.bfloat16, 5),
]


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_forward_matches_row_by_row_oracle(case):
    T, d, E, k, d_ff, tau, renorm, cap, policy, dt, chunk = case
    p = _layer(T, d, E, d_ff, 1, dt)
    kw = dict(k=k, tau=tau, renormalize=renorm, cap_num=cap[0], cap_den=cap[1],
              drop_policy=policy)
    ref = orc.forward(p["x"], p["w_router"], p["bias"], p["w_gate"], p["w_up"], p["w_down"],
                      want_h=True, **kw)
    assert ref["n_kept"] < T * k or cap[1] == 0
    seen = np.zeros(ref["n_kept"], dtype=bool)
    slot_of_row = np.full(ref["n_kept"], -1)
    kept = ref["row_of"] >= 0
    slot_of_row[ref["row_of"][kept]] = np.nonzero(kept.ravel())[0]

    def on_block(e, r0, r1, h, o):
        assert (ref["idx"].ravel()[slot_of_row[r0:r1]] == e).all()
        _close(h, ref["h_slots"][slot_of_row[r0:r1]])
        _close(o, ref["o_slots"][slot_of_row[r0:r1]])
        seen[r0:r1] = True

    y = by_expert.forward_full(p["x"], p["w_gate"], p["w_up"], p["w_down"], ref["offset"],
                               ref["token_of_row"], ref["row_of"], ref["gate"], T, chunk=chunk,
                               on_block=on_block)
    assert seen.all()
    _close(y, ref["y"])
    dropped = ~kept.any(1)
    assert (y[dropped] == 0).all()


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_backward_matches_row_by_row_oracle(case):
    T, d, E, k, d_ff, tau, renorm, cap, policy, dt, chunk = case
    p = _layer(T, d, E, d_ff, 2, dt)
    dy = torch.randn((T, d), generator=torch.Generator().manual_seed(9)).double().numpy()
    kw = dict(k=k, tau=tau, renormalize=renorm, cap_num=cap[0], cap_den=cap[1],
              drop_policy=policy)
    ref = orc.backward(p["x"], p["w_router"], p["bias"], p["w_gate"], p["w_up"], p["w_down"],
                       dy, **kw)
    dsp = orc.dispatch(ref["idx"], E, ref["C"], policy)
    got = by_expert.backward(p["x"], p["w_router"], p["w_gate"], p["w_up"], p["w_down"], dy,
                             logits=ref["logits"], idx=ref["idx"], gate=ref["gate"],
                             row_of=dsp["row_of"], offset=dsp["offset"],
                             token_of_row=dsp["token_of_row"], tau=tau, renormalize=renorm,
                             chunk=chunk)
    for name in ("dx", "dgate", "dw_router", "dbias", "dw_gate", "dw_up", "dw_down"):
        _close(got[name], ref[name])
    # expert by expert through the callback: the same values
    per = {}
    got2 = by_expert.backward(p["x"], p["w_router"], p["w_gate"], p["w_up"], p["w_down"], dy,
                              logits=ref["logits"], idx=ref["idx"], gate=ref["gate"],
                              row_of=dsp["row_of"], offset=dsp["offset"],
                              token_of_row=dsp["token_of_row"], tau=tau, renormalize=renorm,
                              chunk=chunk, on_expert=lambda e, g: per.__setitem__(e, g))
    assert sorted(per) == list(range(E)) and "dw_gate" not in got2
    for name in ("dw_gate", "dw_up", "dw_down"):
        _close(np.stack([per[e][name] for e in range(E)]), ref[name])


def test_router_backward_gives_the_router_gradients_of_the_full_backward():
    T, d, E, k, d_ff = 64, 24, 6, 2, 32
    p = _layer(T, d, E, d_ff, 3)
    dy = torch.randn((T, d), generator=torch.Generator().manual_seed(4)).double().numpy()
    for renorm, tau in ((True, 0.4), (False, 1.3)):
        ref = orc.backward(p["x"], p["w_router"], p["bias"], p["w_gate"], p["w_up"],
                           p["w_down"], dy, k=k, tau=tau, renormalize=renorm, cap_num=1,
                           cap_den=1)
        dl = orc.router_backward(ref["logits"], ref["idx"], ref["gate"], ref["dgate"], tau, renorm)
        _close(dl.sum(0), ref["dbias"])
        _close(p["x"].double().numpy().T @ dl, ref["dw_router"])
        # the softmax backward sums to zero over the experts of every token
        assert np.abs(dl.sum(1)).max() <= 1e-12 * np.abs(dl).max()


def test_widen_is_exact_for_bf16_patterns():
    t = torch.randn(1000).bfloat16()
    raw = t.view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(by_expert.widen(raw), t.double().numpy())
    np.testing.assert_array_equal(by_expert.widen(t), t.double().numpy())

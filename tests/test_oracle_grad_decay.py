"""Pins for the float64 gradient oracle of the per-token-decay operator
(oracle/wkv_grad.py, wkv_dd_backward_direct).

Checked against central finite differences of the forward oracle
wkv_dd_direct (itself pinned against the mpmath brute force in
test_oracle_decay.py) for every input element of small cases, rate by rate;
against the constant-decay gradient oracle when every rate is the same (the
rate gradients then add up to the constant w's); and against properties of
the operator: an output does not depend on the rates of its own or later
steps, nor (from the empty state) on the rate of step 0, and shifting every
key and the initial max_exp together changes nothing. Planted mistakes in
the oracle's source (run on the CPU) must fail the finite-difference pin."""

import inspect

import numpy as np
import pytest

import oracle.wkv_grad as G
from oracle import wkv_backward_direct, wkv_dd_backward_direct, wkv_dd_direct


def _case(seed, B, T, C, kscale=1.0, with_state=False):
    g = np.random.default_rng([41, seed])
    w = np.exp(g.uniform(np.log(0.05), np.log(3.0), (B, T, C)))
    u = g.normal(0, 1, C)
    k = g.normal(0, kscale, (B, T, C))
    v = g.normal(0, 1, (B, T, C))
    gout = g.normal(0, 1, (B, T, C))
    s0 = None
    if with_state:
        s0 = np.stack([g.normal(0, 1, (B, C)), g.uniform(0.5, 2.0, (B, C)),
                       g.normal(0, 2, (B, C))])
    gs = np.stack([g.normal(0, 1, (B, C)), g.normal(0, 1, (B, C)), np.zeros((B, C))])
    return w, u, k, v, gout, s0, gs


def _loss(w, u, k, v, gout, s0, gs, m_star):
    out, st = wkv_dd_direct(w, u, k, v, s0)
    val = (gout * out).sum()
    if gs is not None:
        # the state term with the representation held at m_star
        scale = np.exp(st[2] - m_star)
        val += (gs[0] * st[0] * scale).sum() + (gs[1] * st[1] * scale).sum()
    return val


def _fd_check(w, u, k, v, gout, s0, gs, backward=wkv_dd_backward_direct, h=1e-6):
    """Largest |analytic - finite difference| over every input element,
    relative to the size of the gradients."""
    m_star = st_out = None
    if gs is not None:
        _, st_out = wkv_dd_direct(w, u, k, v, s0)
        m_star = st_out[2]
    gw, gu, gk, gv, gs0 = backward(w, u, k, v, gout, s0, gs, st_out)
    args = {"w": w, "u": u, "k": k, "v": v}
    if s0 is not None:
        args["s0"] = s0
    analytic = {"w": gw, "u": gu, "k": gk, "v": gv, "s0": gs0}
    worst = 0.0
    for name, arr in args.items():
        for idx in np.ndindex(arr.shape):
            plus = {n: a.copy() for n, a in args.items()}
            minus = {n: a.copy() for n, a in args.items()}
            plus[name][idx] += h
            minus[name][idx] -= h
            lp = _loss(plus["w"], plus["u"], plus["k"], plus["v"], gout, plus.get("s0"), gs,
                       m_star)
            lm = _loss(minus["w"], minus["u"], minus["k"], minus["v"], gout, minus.get("s0"), gs,
                       m_star)
            worst = max(worst, abs((lp - lm) / (2 * h) - analytic[name][idx]))
    scale = max(np.abs(gk).max(), np.abs(gv).max(), 1e-3)
    return worst / scale


@pytest.mark.parametrize("with_state", [False, True])
@pytest.mark.parametrize("with_gstate", [False, True])
@pytest.mark.parametrize("kscale", [1.0, 8.0])
def test_gradients_match_finite_differences(with_state, with_gstate, kscale):
    w, u, k, v, gout, s0, gs = _case(int(kscale) * 4 + 2 * with_state + with_gstate, 2, 5, 2,
                                     kscale, with_state)
    err = _fd_check(w, u, k, v, gout, s0, gs if with_gstate else None)
    assert err < 1e-7, err


def test_gradients_match_finite_differences_longer_sequence():
    w, u, k, v, gout, s0, gs = _case(77, 1, 11, 2, 2.0, True)
    assert _fd_check(w, u, k, v, gout, s0, gs) < 1e-7


@pytest.mark.parametrize("with_state", [False, True])
def test_constant_rates_give_the_constant_decay_gradients(with_state):
    """With w_t = w for every t the operator is the constant-decay one, so
    its gradients are wkv_backward_direct's, the rate gradients summed over
    batch rows and positions giving dL/dw."""
    w, u, k, v, gout, s0, gs = _case(31 + with_state, 3, 9, 4, 2.0, with_state)
    wc = w[0, 0]
    wt = np.broadcast_to(wc, k.shape).copy()
    _, st = wkv_dd_direct(wt, u, k, v, s0)
    got = wkv_dd_backward_direct(wt, u, k, v, gout, s0, gs, st)
    ref = wkv_backward_direct(wc, u, k, v, gout, s0, gs, st)
    assert np.allclose(got[0].sum(axis=(0, 1)), ref[0], rtol=1e-10, atol=1e-12)
    for a, b in zip(got[1:], ref[1:]):
        assert np.allclose(a, b, rtol=1e-10, atol=1e-12)


def test_outputs_do_not_depend_on_own_or_later_rates():
    """out_t holds the rates of steps 0 .. t-1 only, and from the empty state
    no term holds step 0's rate: with dL/dout nonzero at t0 alone, dL/dw_j
    is exactly zero for j >= t0 and for j = 0, and nonzero in between."""
    w, u, k, v, gout, _, _ = _case(44, 2, 10, 3)
    t0 = 6
    g = np.zeros_like(gout)
    g[:, t0] = gout[:, t0]
    gw, *_ = wkv_dd_backward_direct(w, u, k, v, g)
    assert np.all(gw[:, t0:] == 0.0)
    assert np.all(gw[:, 0] == 0.0)
    assert np.all(np.abs(gw[:, 1:t0]) > 0.0)


def test_key_shift_invariance_of_gradients():
    """out is unchanged when every key and the initial max_exp move together,
    so per lane sum_t dL/dk_t + dL/dm0 = 0."""
    for with_state in (False, True):
        w, u, k, v, gout, s0, _ = _case(5, 3, 9, 4, 3.0, with_state)
        gw, gu, gk, gv, gs0 = wkv_dd_backward_direct(w, u, k, v, gout, s0)
        total = gk.sum(axis=1) + gs0[2]
        assert np.abs(total).max() < 1e-12 * max(1.0, np.abs(gk).max())


MUTANTS = [
    # the rates collected one step off
    ("            gw[:, 1:upto] -= np.cumsum(dx, axis=1)[:, :upto - 1]",
     "            gw[:, :upto - 1] -= np.cumsum(dx, axis=1)[:, :upto - 1]"),
    # the initial state's decay left out of the rate gradient
    ("            gw[:, :t] -= dx_init[:, None, :]", "            gw[:, :t] -= 0 * dx_init[:, None, :]"),
    # final-state term: token i decayed by its own step's rate too
    ("        e_tok = np.exp(k - (cum[:, T][:, None] - cum[:, idx + 1]) - m_out[:, None])",
     "        e_tok = np.exp(k - (cum[:, T][:, None] - cum[:, idx]) - m_out[:, None])"),
]


@pytest.mark.parametrize("old,new", MUTANTS)
def test_planted_mistakes_fail_the_finite_difference_pin(old, new):
    src = inspect.getsource(G)
    assert old in src
    ns = {"__name__": "mutant"}
    code = (src.replace(old, new)
            .replace("from .wkv_oracle import", "from oracle.wkv_oracle import")
            .replace("from .wkv_decay import", "from oracle.wkv_decay import"))
    exec(compile(code, "mutant", "exec"), ns)
    w, u, k, v, gout, s0, gs = _case(21, 1, 5, 2, 1.0, True)
    assert _fd_check(w, u, k, v, gout, s0, gs, backward=ns["wkv_dd_backward_direct"]) > 1e-4

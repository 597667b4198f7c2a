"""Pins for the float64 gradient oracle (oracle/wkv_grad.py).

The gradients are checked against central finite differences of the forward
oracle wkv_direct (itself pinned against the mpmath brute force in
test_oracle.py), for every input element of small cases, and against
invariants of the operator that do not depend on how the gradient is
computed: the output does not change when every key and the initial state's
max_exp move by the same amount, it is homogeneous of degree one in (v, n0),
and it does not depend on w for T <= 2 from the empty state. Planted mistakes
in the oracle's source (run on the CPU) must fail the finite-difference
check. The receptance gate's sigmoid is checked against scipy's, the gated
output at the gate's special values (fully open, r = 0), and the gated
gradients (including dL/dr) by finite differences of the gated forward."""

import inspect

import numpy as np
import pytest

import oracle.wkv_grad as G
from oracle import wkv_backward_direct, wkv_direct


def _case(seed, B, T, C, kscale=1.0, with_state=False):
    g = np.random.default_rng([31, seed])
    w = np.exp(g.uniform(np.log(0.05), np.log(3.0), C))
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
    out, st = wkv_direct(w, u, k, v, s0)
    val = (gout * out).sum()
    if gs is not None:
        # the state term with the representation held at m_star
        scale = np.exp(st[2] - m_star)
        val += (gs[0] * st[0] * scale).sum() + (gs[1] * st[1] * scale).sum()
    return val


def _fd_check(w, u, k, v, gout, s0, gs, backward=wkv_backward_direct, h=1e-6):
    """Largest |analytic - finite difference| over every input element,
    relative to the size of the gradients."""
    m_star = None
    st_out = None
    if gs is not None:
        _, st_out = wkv_direct(w, u, k, v, s0)
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
            lp = _loss(plus["w"], plus["u"], plus["k"], plus["v"], gout, plus.get("s0"), gs, m_star)
            lm = _loss(minus["w"], minus["u"], minus["k"], minus["v"], gout, minus.get("s0"), gs,
                       m_star)
            fd = (lp - lm) / (2 * h)
            worst = max(worst, abs(fd - analytic[name][idx]))
    scale = max(np.abs(gk).max(), np.abs(gv).max(), 1e-3)
    return worst / scale


@pytest.mark.parametrize("with_state", [False, True])
@pytest.mark.parametrize("with_gstate", [False, True])
@pytest.mark.parametrize("kscale", [1.0, 8.0])
def test_gradients_match_finite_differences(with_state, with_gstate, kscale):
    w, u, k, v, gout, s0, gs = _case(int(kscale) * 4 + 2 * with_state + with_gstate, 2, 5, 3,
                                     kscale, with_state)
    err = _fd_check(w, u, k, v, gout, s0, gs if with_gstate else None)
    assert err < 1e-7, err


def test_gradients_match_finite_differences_longer_sequence():
    w, u, k, v, gout, s0, gs = _case(77, 1, 12, 2, 2.0, True)
    assert _fd_check(w, u, k, v, gout, s0, gs) < 1e-7


def test_key_shift_invariance_of_gradients():
    """out is unchanged when every key and the initial max_exp move together,
    so per lane sum_t dL/dk_t + dL/dm0 = 0."""
    for with_state in (False, True):
        w, u, k, v, gout, s0, _ = _case(5, 3, 9, 4, 3.0, with_state)
        gw, gu, gk, gv, gs0 = wkv_backward_direct(w, u, k, v, gout, s0)
        total = gk.sum(axis=1) + gs0[2]
        assert np.abs(total).max() < 1e-12 * max(1.0, np.abs(gk).max())


def test_value_homogeneity_of_gradients():
    """out is homogeneous of degree one in (v, n0): per lane
    sum_t v_t dL/dv_t + n0 dL/dn0 = sum_t gout_t out_t."""
    w, u, k, v, gout, s0, _ = _case(6, 2, 11, 3, 1.5, True)
    gw, gu, gk, gv, gs0 = wkv_backward_direct(w, u, k, v, gout, s0)
    out, _ = wkv_direct(w, u, k, v, s0)
    lhs = (v * gv).sum(axis=1) + s0[0] * gs0[0]
    rhs = (gout * out).sum(axis=1)
    assert np.allclose(lhs, rhs, rtol=1e-12, atol=1e-12)


def test_no_decay_gradient_for_two_tokens():
    """From the empty state out_1 and out_2 do not involve w (the newest past
    token is never decayed), so dL/dw = 0 for T <= 2."""
    for T in (1, 2):
        w, u, k, v, gout, _, _ = _case(8 + T, 2, T, 5)
        gw, *_ = wkv_backward_direct(w, u, k, v, gout)
        assert np.abs(gw).max() == 0.0


def test_first_token_gradients_closed_form():
    """T = 1 from the empty state: out_1 = v_1, so dL/dv_1 = gout_1 and every
    other gradient is zero."""
    w, u, k, v, gout, _, _ = _case(12, 2, 1, 4)
    gw, gu, gk, gv, gs0 = wkv_backward_direct(w, u, k, v, gout)
    assert np.array_equal(gv, gout)
    assert np.abs(gk).max() == 0 and np.abs(gu).max() == 0 and np.abs(gw).max() == 0


MUTANTS = [
    # decay age off by one in the w gradient
    ("gw += (dx_past * -age).sum(axis=1)", "gw += (dx_past * -(age + 1)).sum(axis=1)"),
    # the current token's own term dropped from dL/dk
    ("gk[:, t] += dx_cur", "gk[:, t] += 0 * dx_cur"),
    # wrong sign on the denominator part of the initial state's gradient
    ("gd0 += -gt * y * r_init", "gd0 += gt * y * r_init"),
    # final-state term: the denominator gradient dropped from dL/dk
    ("dx_tok = e_tok * (gn[:, None] * v + gd[:, None])", "dx_tok = e_tok * (gn[:, None] * v)"),
    # bonus applied to the value gradient of past tokens too
    ("gv[:, :t] += gt[:, None] * r_past", "gv[:, :t] += gt[:, None] * r_past * np.exp(u)"),
]


@pytest.mark.parametrize("old,new", MUTANTS)
def test_planted_mistakes_fail_the_finite_difference_pin(old, new):
    src = inspect.getsource(G)
    assert old in src
    ns = {"__name__": "mutant"}
    code = src.replace(old, new).replace("from .wkv_oracle import empty_state",
                                         "from oracle.wkv_oracle import empty_state")
    exec(compile(code, "mutant", "exec"), ns)
    w, u, k, v, gout, s0, gs = _case(21, 1, 4, 2, 1.0, True)
    assert _fd_check(w, u, k, v, gout, s0, gs, backward=ns["wkv_backward_direct"]) > 1e-4


# ---------------------------------------------------------------- the gate

def test_sigmoid_matches_scipy():
    import scipy.special

    from oracle import sigmoid

    x = np.concatenate([np.linspace(-50, 50, 1001), [-800.0, 800.0, 0.0]])
    assert np.allclose(sigmoid(x), scipy.special.expit(x), rtol=1e-15, atol=1e-300)


def test_gate_special_values():
    """r -> +inf passes the WKV output through, r = 0 halves it."""
    from oracle import wkv_gated

    w, u, k, v, _, s0, _ = _case(90, 2, 7, 3, 1.0, True)
    plain, st = wkv_direct(w, u, k, v, s0)
    open_gate, st2 = wkv_gated(w, u, k, v, np.full(k.shape, 1e3), s0)
    half, _ = wkv_gated(w, u, k, v, np.zeros(k.shape), s0)
    assert np.array_equal(open_gate, plain) and np.array_equal(st2, st)
    assert np.array_equal(half, 0.5 * plain)


@pytest.mark.parametrize("with_state", [False, True])
def test_gated_gradients_match_finite_differences(with_state):
    from oracle import wkv_gated, wkv_gated_backward_direct

    w, u, k, v, gout, s0, _ = _case(91 + with_state, 2, 6, 3, 2.0, with_state)
    r = np.random.default_rng([92]).normal(0, 2, k.shape)
    gw, gu, gk, gv, gs0, gr = wkv_gated_backward_direct(w, u, k, v, r, gout, s0)
    args = {"w": w, "u": u, "k": k, "v": v, "r": r}
    if s0 is not None:
        args["s0"] = s0
    analytic = {"w": gw, "u": gu, "k": gk, "v": gv, "r": gr, "s0": gs0}

    def loss(a):
        out, _ = wkv_gated(a["w"], a["u"], a["k"], a["v"], a["r"], a.get("s0"))
        return (gout * out).sum()

    h, worst = 1e-6, 0.0
    for name, arr in args.items():
        for idx in np.ndindex(arr.shape):
            plus = {n: x.copy() for n, x in args.items()}
            minus = {n: x.copy() for n, x in args.items()}
            plus[name][idx] += h
            minus[name][idx] -= h
            fd = (loss(plus) - loss(minus)) / (2 * h)
            worst = max(worst, abs(fd - analytic[name][idx]))
    assert worst / max(np.abs(gk).max(), np.abs(gr).max()) < 1e-7

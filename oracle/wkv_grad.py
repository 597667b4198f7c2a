"""Float64 CPU oracle for the gradients of the WKV operator (its backward pass).

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module. It shares no code with the HIP library.

What is computed
----------------
The forward operator is the one of the page "Linear attention without writing a
CUDA kernel", section "The recurrence" (the wkv_t equation): for every lane
(b, c) and position t,

    out_t = Num_t / Den_t,   Num_t = sum_j a_j e^{x_j},   Den_t = sum_j b_j e^{x_j}

over the terms j present at position t: the initial state (exponent
m0 - t w, coefficients n0 and d0), every past token i < t (exponent
k_i - (t-1-i) w, coefficients v_i and 1) and the current token (exponent
u + k_t, coefficients v_t and 1). The page trains its model through this
operator (page "MicroRWKV", and the training form named on the page "RWKV-v6
Architecture: Attention-Free Linear Transformers", section on architectural
duality), so its gradients are the derivatives of this ratio. By the quotient
rule, for one position t:

    d out_t / d x_j = e^{x_j} (a_j - out_t b_j) / Den_t
    d out_t / d a_j = e^{x_j} / Den_t
    d out_t / d b_j = -out_t e^{x_j} / Den_t

and every input reaches out_t only through the x_j, a_j, b_j above (k_i through
x_i with derivative 1, w through x_i with derivative -(t-1-i) and through the
initial state's exponent with -t, u through the current token's exponent, v_i
through a_i, n0 and d0 through the initial state's coefficients and m0 through
its exponent). The gradients here are these chain-rule sums written out term by
term for every (t, j) pair: O(T^2) per lane, small inputs only.

The final state (N_T, D_T) = (sum_j a_j e^{x_j}, sum_j b_j e^{x_j}) over the
terms left after the last token (token i decayed T-1-i times, the initial state
T times, no bonus) is an output too. Its upstream gradient is given, like the
state itself, as three planes (g_num, g_den, g_max) for the state
(num, den, max_exp) = (N e^-m, D e^-m, m) that the forward returned, so the
gradient with respect to the true sums is g_num e^-m and g_den e^-m. g_max is
not used: (num, den, max_exp) and (num e^s, den e^s, max_exp - s) are the same
state, so for any loss that depends on the state itself g_max equals
num g_num + den g_den and carries nothing new.

The gradient of the initial state is returned for the three planes as given:
(d/dn0, d/dd0, d/dm0), where d/dm0 = n0 d/dn0 + d0 d/dd0.
"""

from __future__ import annotations

import numpy as np

from .wkv_oracle import empty_state, sigmoid, wkv_direct


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def wkv_backward_direct(w, u, k, v, gout, state_in=None, gstate_out=None, state_out=None):
    """Gradients of sum(gout * out) + <gstate_out, state_out> (see module
    docstring) with respect to w (C,), u (C,), k (B, T, C), v (B, T, C) and the
    initial state (3, B, C).

    gout: (B, T, C) upstream gradient of out. gstate_out, state_out: both
    (3, B, C) or both None; state_out is the state the forward returned (only
    its max_exp plane is used, to turn g_num, g_den into gradients of the true
    sums). Returns (gw, gu, gk, gv, gstate_in); gstate_in is all zeros when
    state_in is None (the empty state is a constant)."""
    w, u, k, v, g = _f64(w), _f64(u), _f64(k), _f64(v), _f64(gout)
    B, T, C = k.shape
    if g.shape != k.shape or v.shape != k.shape:
        raise ValueError("k, v and gout must all be (B, T, C)")
    if (gstate_out is None) != (state_out is None):
        raise ValueError("gstate_out and state_out go together")
    have_init = state_in is not None
    s0 = empty_state(B, C) if state_in is None else _f64(state_in)
    n0, d0, m0 = s0

    gw = np.zeros((B, C))
    gu = np.zeros((B, C))
    gk = np.zeros((B, T, C))
    gv = np.zeros((B, T, C))
    gn0 = np.zeros((B, C))
    gd0 = np.zeros((B, C))
    gm0 = np.zeros((B, C))

    for t in range(T):
        # exponents and coefficients of every term present at position t
        past = np.arange(t)
        age = (t - 1 - past)[None, :, None].astype(np.float64)
        x_past = k[:, :t] - age * w
        x_cur = u + k[:, t]
        x_init = m0 - t * w
        top = np.maximum(x_cur, x_init)
        if t > 0:
            top = np.maximum(top, x_past.max(axis=1))
        e_past = np.exp(x_past - top[:, None])
        e_cur = np.exp(x_cur - top)
        e_init = np.exp(x_init - top) if have_init else np.zeros((B, C))
        den = e_past.sum(axis=1) + e_cur + e_init * d0
        num = (e_past * v[:, :t]).sum(axis=1) + e_cur * v[:, t] + e_init * n0
        y = num / den
        gt = g[:, t]
        # e^{x_j} / Den_t for every term, with the common factor e^{top} cancelled
        r_past = e_past / den[:, None]
        r_cur = e_cur / den
        r_init = e_init / den

        # past tokens i < t
        dx_past = gt[:, None] * r_past * (v[:, :t] - y[:, None])
        gk[:, :t] += dx_past
        gv[:, :t] += gt[:, None] * r_past
        gw += (dx_past * -age).sum(axis=1)
        # the current token
        dx_cur = gt * r_cur * (v[:, t] - y)
        gk[:, t] += dx_cur
        gv[:, t] += gt * r_cur
        gu += dx_cur
        # the initial state
        if have_init:
            dx_init = gt * r_init * (n0 - y * d0)
            gm0 += dx_init
            gw += dx_init * -t
            gn0 += gt * r_init
            gd0 += -gt * y * r_init

    if gstate_out is not None:
        gn, gd = _f64(gstate_out)[0], _f64(gstate_out)[1]
        m_out = _f64(state_out)[2]
        # N_T = n0 e^{m0 - T w} + sum_i e^{k_i - (T-1-i) w} v_i, D_T likewise;
        # dL/dN_T = gn e^{-m_out}, dL/dD_T = gd e^{-m_out}
        age = (T - 1 - np.arange(T))[None, :, None].astype(np.float64)
        e_tok = np.exp(k - age * w - m_out[:, None])
        gv += gn[:, None] * e_tok
        dx_tok = e_tok * (gn[:, None] * v + gd[:, None])
        gk += dx_tok
        gw += (dx_tok * -age).sum(axis=1)
        if have_init:
            e0 = np.exp(m0 - T * w - m_out)
            gn0 += gn * e0
            gd0 += gd * e0
            dx0 = e0 * (gn * n0 + gd * d0)
            gm0 += dx0
            gw += dx0 * -T

    gstate_in = np.stack([gn0, gd0, gm0])
    return gw.sum(axis=0), gu.sum(axis=0), gk, gv, gstate_in


# ---------------------------------------------------------------------------
# The receptance gate on the output (see wkv_oracle.wkv_gated).
# ---------------------------------------------------------------------------

def wkv_gated_backward_direct(w, u, k, v, r, gout, state_in=None, gstate_out=None,
                              state_out=None):
    """Gradients of sum(gout * sigmoid(r) * wkv) (+ the final-state term of
    wkv_backward_direct): by the product rule dL/dr = gout * wkv * s (1 - s)
    with s = sigmoid(r), and the WKV gradients are those of the ungated
    operator for the upstream gradient gout * s. Returns
    (gw, gu, gk, gv, gstate_in, gr). wkv is the forward oracle's output."""
    s = sigmoid(r)
    y, _ = wkv_direct(w, u, k, v, state_in)
    g = _f64(gout)
    gw, gu, gk, gv, gs = wkv_backward_direct(w, u, k, v, g * s, state_in, gstate_out, state_out)
    return gw, gu, gk, gv, gs, g * y * s * (1.0 - s)


# ---------------------------------------------------------------------------
# Per-token (data-dependent) decay (see wkv_decay.wkv_dd_direct).
# ---------------------------------------------------------------------------

def wkv_dd_backward_direct(w, u, k, v, gout, state_in=None, gstate_out=None, state_out=None):
    """Gradients of sum(gout * out) (+ the final-state term, as in
    wkv_backward_direct) for the operator with a decay rate per token,
    w (B, T, C). The terms are those of wkv_decay.wkv_dd_direct: at output t
    the initial state has exponent m0 - sum_{j<t} w_j, past token i < t
    exponent k_i - sum_{j=i+1}^{t-1} w_j, the current token u + k_t; the final
    state holds token i at k_i - sum_{j=i+1}^{T-1} w_j and the initial state at
    m0 - sum_{j<T} w_j. The quotient-rule derivatives of wkv_backward_direct
    apply unchanged; a rate w_j enters (with derivative -1) the exponent of
    every term whose decay range contains step j. Term by term, O(T^2) per
    lane. Returns (gw (B, T, C), gu (C,), gk, gv, gstate_in)."""
    from .wkv_decay import _check

    w, u, k, v, s0 = _check(w, u, k, v, state_in)
    g = _f64(gout)
    B, T, C = k.shape
    if g.shape != k.shape:
        raise ValueError("gout must be (B, T, C)")
    if (gstate_out is None) != (state_out is None):
        raise ValueError("gstate_out and state_out go together")
    have_init = state_in is not None
    n0, d0, m0 = s0
    # cum[:, t] = sum_{j<t} w_j; the rates of steps lo .. hi-1 are cum[hi] - cum[lo]
    cum = np.concatenate([np.zeros((B, 1, C)), np.cumsum(w, axis=1)], axis=1)

    gw = np.zeros((B, T, C))
    gu = np.zeros((B, C))
    gk = np.zeros((B, T, C))
    gv = np.zeros((B, T, C))
    gn0 = np.zeros((B, C))
    gd0 = np.zeros((B, C))
    gm0 = np.zeros((B, C))

    def to_rates(dx, upto):
        """Terms 0 .. n-1 of past tokens i whose exponents hold the rates of
        steps i+1 .. upto-1: rate j collects -dx_i from every token i < j,
        i.e. minus the running sum of dx up to token j-1."""
        if upto > 1:
            gw[:, 1:upto] -= np.cumsum(dx, axis=1)[:, :upto - 1]

    for t in range(T):
        past = np.arange(t)
        x_past = k[:, :t] - (cum[:, t][:, None] - cum[:, past + 1])   # steps i+1 .. t-1
        x_cur = u + k[:, t]
        x_init = m0 - cum[:, t]                                        # steps 0 .. t-1
        top = np.maximum(x_cur, x_init)
        if t > 0:
            top = np.maximum(top, x_past.max(axis=1))
        e_past = np.exp(x_past - top[:, None])
        e_cur = np.exp(x_cur - top)
        e_init = np.exp(x_init - top) if have_init else np.zeros((B, C))
        den = e_past.sum(axis=1) + e_cur + e_init * d0
        num = (e_past * v[:, :t]).sum(axis=1) + e_cur * v[:, t] + e_init * n0
        y = num / den
        gt = g[:, t]
        r_past = e_past / den[:, None]
        r_cur = e_cur / den
        r_init = e_init / den

        dx_past = gt[:, None] * r_past * (v[:, :t] - y[:, None])
        gk[:, :t] += dx_past
        gv[:, :t] += gt[:, None] * r_past
        to_rates(dx_past, t)
        dx_cur = gt * r_cur * (v[:, t] - y)
        gk[:, t] += dx_cur
        gv[:, t] += gt * r_cur
        gu += dx_cur
        if have_init:
            dx_init = gt * r_init * (n0 - y * d0)
            gm0 += dx_init
            gw[:, :t] -= dx_init[:, None, :]
            gn0 += gt * r_init
            gd0 += -gt * y * r_init

    if gstate_out is not None:
        gn, gd = _f64(gstate_out)[0], _f64(gstate_out)[1]
        m_out = _f64(state_out)[2]
        idx = np.arange(T)
        e_tok = np.exp(k - (cum[:, T][:, None] - cum[:, idx + 1]) - m_out[:, None])
        gv += gn[:, None] * e_tok
        dx_tok = e_tok * (gn[:, None] * v + gd[:, None])
        gk += dx_tok
        to_rates(dx_tok, T)
        if have_init:
            e0 = np.exp(m0 - cum[:, T] - m_out)
            gn0 += gn * e0
            gd0 += gd * e0
            dx0 = e0 * (gn * n0 + gd * d0)
            gm0 += dx0
            gw -= dx0[:, None, :]

    gstate_in = np.stack([gn0, gd0, gm0])
    return gw, gu.sum(axis=0), gk, gv, gstate_in

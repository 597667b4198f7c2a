"""Float64 oracle for the WKV operator with a data-dependent (per-token) decay.

TEST INFRASTRUCTURE, like the rest of this package: only the test suite, the
smoke check and the benchmark's CPU-baseline leg may import it. It shares no
code with the HIP library.

What is computed
----------------
Source: the page "RWKV-v6 Architecture: Attention-Free Linear Transformers",
section "The Core Components of the RWKV-v6 Time-Mixing Block", items
"Dynamic Data-Dependent Decay" and "Matrix-Valued Hidden State". The decay
becomes a vector w_t computed from each token, and the recurrence multiplies
the state carried in from position t-1 by step t's decay before step t's own
key-value term is added.

Applied to the vector-state operator of the page "Linear attention without
writing a CUDA kernel" (section "The recurrence"; see wkv_oracle.py), with the
decay given per token and channel as a positive rate:

* w has k's shape (B, T, C); step t multiplies the carried state by
  exp(-w_t). (The first page writes its decay as the factor itself,
  exp(-exp(.)) in (0, 1); the rate here is the inner exp(.), the same
  parametrisation as the constant-decay operator's w.)
* Output at position t (0-based): the state before step t, i.e. every past
  token i < t decayed by the rates of the steps after it up to t-1,
      exp(k_i - sum_{j=i+1}^{t-1} w_j),
  the initial state decayed by sum_{j=0}^{t-1} w_j, and the current token
  with the bonus exp(u + k_t), as in the constant-decay operator.
* State after the last token: token i decayed by sum_{j=i+1}^{T-1} w_j, the
  initial state by sum_{j=0}^{T-1} w_j.

With w_t equal to a constant w this is exactly the constant-decay operator:
the sums become (t-1-i) w and t w.

Every function works in float64 on copies of its inputs.
"""

from __future__ import annotations

import numpy as np

from .wkv_oracle import empty_state


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _check(w, u, k, v, state_in):
    w, u, k, v = _f64(w), _f64(u), _f64(k), _f64(v)
    if k.ndim != 3 or v.shape != k.shape or w.shape != k.shape:
        raise ValueError(f"w, k and v must all be (B, T, C); got {w.shape}, {k.shape}, {v.shape}")
    B, T, C = k.shape
    if u.shape != (C,):
        raise ValueError(f"u must be ({C},); got {u.shape}")
    if state_in is None:
        state_in = empty_state(B, C)
    state_in = _f64(state_in)
    if state_in.shape != (3, B, C):
        raise ValueError(f"state must be (3, {B}, {C}); got {state_in.shape}")
    return w, u, k, v, state_in.copy()


def _decay_between(w, lo, hi):
    """sum_{j=lo}^{hi-1} w_j along axis 1 for every lane: the total rate of
    steps lo .. hi-1 (zero when lo >= hi)."""
    if hi <= lo:
        return np.zeros((w.shape[0], w.shape[2]))
    return w[:, lo:hi].sum(axis=1)


def wkv_dd_direct(w, u, k, v, state_in=None):
    """The operator by its defining sums (O(T^2) per lane, or O(T^3) counting
    the decay sums; small inputs only). Returns (out, state_out) with
    state_out = (N e^-M, D e^-M, M), M the largest exponent left after the last
    token."""
    w, u, k, v, s0 = _check(w, u, k, v, state_in)
    B, T, C = k.shape
    n0, d0, m0 = s0
    out = np.empty((B, T, C))
    for t in range(T):
        exps = np.empty((B, t + 2, C))
        numc = np.empty_like(exps)
        denc = np.empty_like(exps)
        # the initial state has passed steps 0 .. t-1
        exps[:, 0] = m0 - _decay_between(w, 0, t)
        numc[:, 0] = n0
        denc[:, 0] = d0
        # past token i has passed steps i+1 .. t-1
        for i in range(t):
            exps[:, 1 + i] = k[:, i] - _decay_between(w, i + 1, t)
            numc[:, 1 + i] = v[:, i]
            denc[:, 1 + i] = 1.0
        exps[:, t + 1] = u + k[:, t]
        numc[:, t + 1] = v[:, t]
        denc[:, t + 1] = 1.0
        top = exps.max(axis=1, keepdims=True)
        e = np.exp(exps - top)
        out[:, t] = (numc * e).sum(axis=1) / (denc * e).sum(axis=1)
    # state after the last token: the initial state has passed every step,
    # token i the steps after it
    exps = np.empty((B, T + 1, C))
    numc = np.empty_like(exps)
    denc = np.empty_like(exps)
    exps[:, 0] = m0 - _decay_between(w, 0, T)
    numc[:, 0] = n0
    denc[:, 0] = d0
    for i in range(T):
        exps[:, 1 + i] = k[:, i] - _decay_between(w, i + 1, T)
        numc[:, 1 + i] = v[:, i]
        denc[:, 1 + i] = 1.0
    top = exps.max(axis=1)
    e = np.exp(exps - top[:, None])
    state_out = np.stack([(numc * e).sum(axis=1), (denc * e).sum(axis=1), top])
    return out, state_out


def wkv_dd_step_ref(w_t, u, k_t, v_t, state):
    """One decode step with this step's own decay rate w_t (B, C): the output
    mixes the state as it stands with the current token at exp(u + k_t); the
    state is then decayed by exp(-w_t) and the token added at exp(k_t). Each
    mix is taken against the larger exponent, as in wkv_step_ref."""
    w_t, u, k_t, v_t = _f64(w_t), _f64(u), _f64(k_t), _f64(v_t)
    num, den, mx = (_f64(p) for p in state)
    cur = u + k_t
    ref = np.maximum(mx, cur)
    f_past, f_cur = np.exp(mx - ref), np.exp(cur - ref)
    out_t = (f_past * num + f_cur * v_t) / (f_past * den + f_cur)
    decayed = mx - w_t
    ref2 = np.maximum(decayed, k_t)
    g_past, g_cur = np.exp(decayed - ref2), np.exp(k_t - ref2)
    return out_t, np.stack([g_past * num + g_cur * v_t, g_past * den + g_cur, ref2])


def wkv_dd_recurrent(w, u, k, v, state_in=None):
    """The operator over a whole sequence by T successive decode steps
    (wkv_dd_step_ref), step t taking w[:, t]."""
    w, u, k, v, state = _check(w, u, k, v, state_in)
    B, T, C = k.shape
    out = np.empty((B, T, C))
    for t in range(T):
        out[:, t], state = wkv_dd_step_ref(w[:, t], u, k[:, t], v[:, t], state)
    return out, state

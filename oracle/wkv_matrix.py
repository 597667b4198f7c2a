"""Float64 oracle for the matrix-valued-state recurrence.

TEST INFRASTRUCTURE, like the rest of this package: only the test suite, the
smoke check and the benchmark's CPU-baseline leg may import it. It shares no
code with the HIP library.

What is computed
----------------
Source: the page "RWKV-v6 Architecture: Attention-Free Linear Transformers",
section "The Core Components of the RWKV-v6 Time-Mixing Block", item
"Matrix-Valued Hidden State", and the step function of its PyTorch listing
(section "Reference Implementation"). The page's markup of the two equations
is damaged; read together with the listing they say:

* the channels are split into H heads of D = C / H channels (channel
  c = h D + i, the listing's view(B, heads, head_dim));
* every head carries a D x D state S; step t scales row i of the state by
  the decay of channel i and adds the outer product of the key and the
  value: S_t[i][j] = w_t[i] S_{t-1}[i][j] + k_t[i] v_t[j];
* the output is the state after the step applied to the key, gated by the
  sigmoid of the receptance: y_t[i] = sigmoid(r_t[i]) sum_j S_t[i][j] k_t[j].

The decay factor w_t in (0, 1) is given here by its rate, a positive lam with
w = exp(-lam) (the page computes w = exp(-exp(.)); lam is the inner exp), as
for the per-token decay of the vector-state operator. Shapes: r, k, v, lam
are (B, T, C); a state is (B, H, D, D) with S[b, h, i, j]; y is (B, T, C).
The empty state is all zeros.

Every function works in float64 on copies of its inputs.
"""

from __future__ import annotations

import numpy as np

from .wkv_oracle import sigmoid


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _check(lam, k, v, r, H, state_in):
    lam, k, v, r = _f64(lam), _f64(k), _f64(v), _f64(r)
    if k.ndim != 3 or not (lam.shape == v.shape == r.shape == k.shape):
        raise ValueError("lam, k, v, r must all be (B, T, C) of one shape")
    B, T, C = k.shape
    if H <= 0 or C % H:
        raise ValueError(f"C = {C} is not a multiple of H = {H}")
    D = C // H
    if state_in is None:
        state_in = np.zeros((B, H, D, D))
    state_in = _f64(state_in)
    if state_in.shape != (B, H, D, D):
        raise ValueError(f"state must be ({B}, {H}, {D}, {D}); got {state_in.shape}")
    heads = lambda x: x.reshape(B, T, H, D)  # noqa: E731
    return heads(lam), heads(k), heads(v), heads(r), state_in.copy(), D


def wkv6_step_ref(lam_t, k_t, v_t, r_t, H, state):
    """One step of the listing's recurrence for all (batch, head) pairs.
    lam_t, k_t, v_t, r_t: (B, C); state: (B, H, D, D). Returns (y_t, new state)."""
    lam_t, k_t, v_t, r_t = (_f64(x) for x in (lam_t, k_t, v_t, r_t))
    B, C = k_t.shape
    D = C // H
    S = _f64(state)
    w = np.exp(-lam_t).reshape(B, H, D)
    kh, vh, rh = k_t.reshape(B, H, D), v_t.reshape(B, H, D), r_t.reshape(B, H, D)
    S = S * w[..., :, None] + kh[..., :, None] * vh[..., None, :]
    y = sigmoid(rh) * np.einsum("bhij,bhj->bhi", S, kh)
    return y.reshape(B, C), S


def wkv6_recurrent(lam, k, v, r, H, state_in=None):
    """The recurrence over a whole sequence, one step per token."""
    lam4, k4, v4, r4, S, D = _check(lam, k, v, r, H, state_in)
    B, T = k4.shape[:2]
    y = np.empty((B, T, H * D))
    for t in range(T):
        y[:, t], S = wkv6_step_ref(lam4[:, t].reshape(B, -1), k4[:, t].reshape(B, -1),
                                   v4[:, t].reshape(B, -1), r4[:, t].reshape(B, -1), H, S)
    return y, S


def wkv6_direct(lam, k, v, r, H, state_in=None):
    """The same by its sums: the state after step t is the initial state with
    row i scaled by exp(-sum_{tau <= t} lam_tau[i]) plus, for every s <= t, the
    outer product k_s v_s^T with row i scaled by exp(-sum_{s < tau <= t}
    lam_tau[i]); the output applies it to k_t and gates it. Nothing is carried
    from one position to the next (O(T^2) per head)."""
    lam4, k4, v4, r4, S0, D = _check(lam, k, v, r, H, state_in)
    B, T = k4.shape[:2]
    y = np.empty((B, T, H, D))

    def state_after(t):
        # decay of row i from just after step s to the end of step t
        S = S0 * np.exp(-lam4[:, :t + 1].sum(axis=1))[..., :, None]
        for s in range(t + 1):
            f = np.exp(-lam4[:, s + 1:t + 1].sum(axis=1))
            S = S + (f * k4[:, s])[..., :, None] * v4[:, s][..., None, :]
        return S

    S = S0
    for t in range(T):
        S = state_after(t)
        y[:, t] = sigmoid(r4[:, t]) * np.einsum("bhij,bhj->bhi", S, k4[:, t])
    return y.reshape(B, T, H * D), S

"""Pins for the matrix-valued-state oracle (oracle/wkv_matrix.py).

* a 50-digit mpmath evaluation in attention form (oracle/wkv_brute.py,
  wkv6_brute: no state matrix, every output a sum over past tokens of decayed
  key entries times value-key dot products), with and without an initial
  state;
* with no decay and a fully open gate the operator is causal linear
  attention with the keys as queries, the values as keys and the keys as
  values: Y = (M o (K V^T)) K per head, M the causal mask, computed with
  numpy matmul;
* T = 1 from the empty state: y[i] = sigmoid(r[i]) k[i] (v . k);
* heads do not interact: one head run alone gives the same slice;
* a huge decay at one step wipes the state (later outputs equal a fresh run);
* split/resume and the recurrence against the sums;
* homogeneity: y is linear in (v, S0) jointly and of degree two in k from the
  empty state.

Planted mistakes (decay applied to columns instead of rows, the readout
taken before the step, the outer product transposed, the gate dropped) must
each fail the brute-force pin.
"""

import inspect

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st
from scipy.special import expit

import oracle.wkv_matrix as M
from oracle.wkv_brute import wkv6_brute

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def case(seed, B, T, H, D, lam_mu=-1.0):
    g = np.random.default_rng([61, seed])
    C = H * D
    k, v, r = (g.normal(0, 1, (B, T, C)) for _ in range(3))
    lam = np.exp(g.normal(lam_mu, 1.0, (B, T, C)))
    S0 = g.normal(0, 1, (B, H, D, D))
    return lam, k, v, r, S0


def close(a, b, tol=1e-12):
    return np.abs(a - b).max() <= tol * max(1.0, np.abs(b).max())


@settings(max_examples=12, deadline=None)
@given(seed=st.integers(0, 2**31 - 1), T=st.integers(1, 6), H=st.integers(1, 2),
       D=st.integers(1, 4), with_state=st.booleans())
def test_sums_and_recurrence_match_brute_force(seed, T, H, D, with_state):
    lam, k, v, r, S0 = case(seed, 1, T, H, D)
    s0 = S0 if with_state else None
    yb = wkv6_brute(lam, k, v, r, H, s0)
    yd, sd = M.wkv6_direct(lam, k, v, r, H, s0)
    yr, sr = M.wkv6_recurrent(lam, k, v, r, H, s0)
    assert close(yd, yb) and close(yr, yb) and close(sd, sr)


def test_no_decay_open_gate_is_causal_linear_attention():
    B, T, H, D = 2, 9, 3, 4
    lam, k, v, _, _ = case(1, B, T, H, D)
    lam[:] = 0.0
    r = np.full(k.shape, 800.0)  # sigmoid = 1 exactly in float64
    y, _ = M.wkv6_recurrent(lam, k, v, r, H)
    mask = np.tril(np.ones((T, T)))
    for b in range(B):
        for h in range(H):
            K = k[b, :, h * D:(h + 1) * D]
            V = v[b, :, h * D:(h + 1) * D]
            ref = (mask * (K @ V.T)) @ K
            assert close(y[b, :, h * D:(h + 1) * D], ref, 1e-13)


def test_first_token_closed_form():
    lam, k, v, r, _ = case(2, 3, 1, 2, 5)
    y, S = M.wkv6_direct(lam, k, v, r, 2)
    kh, vh = k[:, 0].reshape(3, 2, 5), v[:, 0].reshape(3, 2, 5)
    ref = expit(r[:, 0].reshape(3, 2, 5)) * kh * (kh * vh).sum(axis=-1, keepdims=True)
    assert close(y[:, 0], ref.reshape(3, 10), 1e-15)
    assert close(S, kh[..., :, None] * vh[..., None, :], 1e-15)


def test_heads_are_independent():
    B, T, H, D = 2, 7, 3, 4
    lam, k, v, r, S0 = case(3, B, T, H, D)
    y, S = M.wkv6_recurrent(lam, k, v, r, H, S0)
    h = 1
    sl = slice(h * D, (h + 1) * D)
    y1, S1 = M.wkv6_recurrent(lam[..., sl], k[..., sl], v[..., sl], r[..., sl], 1, S0[:, h:h + 1])
    assert np.array_equal(y1, y[..., sl]) and np.array_equal(S1[:, 0], S[:, h])


def test_huge_decay_wipes_the_state():
    B, T, H, D = 2, 10, 2, 3
    lam, k, v, r, S0 = case(4, B, T, H, D)
    t0 = 4
    lam[:, t0] = 1e4
    y, S = M.wkv6_recurrent(lam, k, v, r, H, S0)
    yf, Sf = M.wkv6_recurrent(lam[:, t0:], k[:, t0:], v[:, t0:], r[:, t0:], H)
    assert close(y[:, t0:], yf, 1e-13) and close(S, Sf, 1e-13)


def test_split_resume_and_direct():
    B, T, H, D = 2, 11, 2, 4
    lam, k, v, r, S0 = case(5, B, T, H, D)
    y, S = M.wkv6_recurrent(lam, k, v, r, H, S0)
    yd, Sd = M.wkv6_direct(lam, k, v, r, H, S0)
    assert close(y, yd) and close(S, Sd)
    for cut in (1, 6):
        y1, S1 = M.wkv6_recurrent(lam[:, :cut], k[:, :cut], v[:, :cut], r[:, :cut], H, S0)
        y2, S2 = M.wkv6_recurrent(lam[:, cut:], k[:, cut:], v[:, cut:], r[:, cut:], H, S1)
        assert close(np.concatenate([y1, y2], axis=1), y, 1e-13) and close(S2, S, 1e-13)


def test_homogeneity():
    B, T, H, D = 1, 8, 2, 3
    lam, k, v, r, S0 = case(6, B, T, H, D)
    y, _ = M.wkv6_recurrent(lam, k, v, r, H, S0)
    y2, _ = M.wkv6_recurrent(lam, k, 2.5 * v, r, H, 2.5 * S0)
    assert close(y2, 2.5 * y, 1e-13)
    y0, _ = M.wkv6_recurrent(lam, k, v, r, H)
    y3, _ = M.wkv6_recurrent(lam, -1.5 * k, v, r, H)
    assert close(y3, 2.25 * y0, 1e-13)


MUTANTS = [
    # decay applied to the columns of the state instead of its rows
    ("S = S * w[..., :, None] + kh[..., :, None] * vh[..., None, :]",
     "S = S * w[..., None, :] + kh[..., :, None] * vh[..., None, :]"),
    # readout from the state before the step
    ("    S = S * w[..., :, None] + kh[..., :, None] * vh[..., None, :]\n"
     "    y = sigmoid(rh) * np.einsum(\"bhij,bhj->bhi\", S, kh)",
     "    y = sigmoid(rh) * np.einsum(\"bhij,bhj->bhi\", S, kh)\n"
     "    S = S * w[..., :, None] + kh[..., :, None] * vh[..., None, :]"),
    # outer product transposed (v k^T)
    ("kh[..., :, None] * vh[..., None, :]\n    y = ", "vh[..., :, None] * kh[..., None, :]\n    y = "),
    # gate dropped
    ("y = sigmoid(rh) * np.einsum", "y = 1.0 * np.einsum"),
]


@pytest.mark.parametrize("old,new", MUTANTS)
def test_planted_mistakes_fail_the_brute_force_pin(old, new):
    src = inspect.getsource(M)
    assert old in src
    code = src.replace(old, new).replace("from .wkv_oracle import sigmoid",
                                         "from oracle.wkv_oracle import sigmoid")
    ns = {"__name__": "mutant"}
    exec(compile(code, "mutant", "exec"), ns)
    lam, k, v, r, S0 = case(7, 1, 4, 2, 3)
    yb = wkv6_brute(lam, k, v, r, 2, S0)
    y, _ = ns["wkv6_recurrent"](lam, k, v, r, 2, S0)
    assert not close(y, yb, 1e-9)

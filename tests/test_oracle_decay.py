"""Pins for the per-token-decay oracle (oracle/wkv_decay.py).

* the 50-digit mpmath recurrence on the raw sums (oracle/wkv_brute.py,
  wkv_dd_brute: a linear recurrence, not the oracle's sum over tokens) on
  tiny random inputs, with and without an initial state and at extreme keys;
* a constant per-token decay gives the constant-decay operator exactly
  (wkv_direct, itself pinned against its own brute force in test_oracle.py);
* a hand-worked case: keys 0, values (1, 0, 0), u = 0 and decay ln 2 at the
  second step give out = (1, 1/2, 1/5) whatever the first and third decays;
* which decays an output depends on: out_t never depends on w_t or later
  rates, and from the empty state not on w_0 either;
* a huge decay at one step wipes the state: afterwards the outputs are those
  of a fresh run started at that token;
* invariants: the decode steps equal the sums, splitting a sequence and
  passing the state on changes nothing, a constant added to every key changes
  no output, outputs stay inside the range of the values mixed.

Planted mistakes (the decay counted from the token's own step, the initial
state missing a step, the final state missing the last step, half the rate
in a step) must each fail one of these pins.
"""

import inspect

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle.wkv_decay as D
from oracle import canonical, normalised_error, wkv_direct
from oracle.wkv_brute import wkv_dd_brute

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def rand_dd(rng, B, T, C, kscale=1.0):
    k = rng.normal(0.0, kscale, (B, T, C))
    v = rng.normal(0.0, 1.0, (B, T, C))
    w = np.exp(rng.normal(-0.5, 1.2, (B, T, C)))  # rates from ~0.03 to ~10
    u = rng.normal(0.0, 0.5, C)
    return w, u, k, v


def random_state(rng, B, C):
    return np.stack([rng.normal(0, 1, (B, C)), rng.uniform(0.5, 3.0, (B, C)),
                     rng.normal(0, 2, (B, C))])


def state_close(a, b, tol):
    ra, La = canonical(a)
    rb, Lb = canonical(b)
    return bool(np.all(np.abs(ra - rb) <= tol * (np.abs(rb) + 1.0))
                and np.all(np.abs(La - Lb) <= tol * np.maximum(1.0, np.abs(Lb))))


def agree_with_brute(fn, w, u, k, v, s0=None, tol=1e-12):
    ob, sb = wkv_dd_brute(w, u, k, v, s0)
    o, s = fn(w, u, k, v, s0)
    return normalised_error(o, ob, 1.0).max() <= tol and state_close(s, sb, tol)


@settings(max_examples=20, deadline=None)
@given(seed=st.integers(0, 2**31 - 1), T=st.integers(1, 10), C=st.integers(1, 3),
       kscale=st.sampled_from([0.5, 2.0, 20.0]))
def test_direct_and_recurrent_match_brute_force(seed, T, C, kscale):
    rng = np.random.default_rng(seed)
    w, u, k, v = rand_dd(rng, 1, T, C, kscale)
    assert agree_with_brute(D.wkv_dd_direct, w, u, k, v)
    assert agree_with_brute(D.wkv_dd_recurrent, w, u, k, v)


def test_brute_force_with_initial_state():
    rng = np.random.default_rng(3)
    w, u, k, v = rand_dd(rng, 2, 8, 3)
    s0 = random_state(rng, 2, 3)
    assert agree_with_brute(D.wkv_dd_direct, w, u, k, v, s0)
    assert agree_with_brute(D.wkv_dd_recurrent, w, u, k, v, s0)


@pytest.mark.parametrize("kmag", [60.0, 88.0])
def test_extreme_keys(kmag):
    rng = np.random.default_rng(4)
    w, u, _, v = rand_dd(rng, 1, 16, 3)
    k = rng.choice([-kmag, kmag, 0.0], size=(1, 16, 3))
    for fn in (D.wkv_dd_direct, D.wkv_dd_recurrent):
        o, s = fn(w, u, k, v)
        assert np.isfinite(o).all() and np.isfinite(s).all()
        assert agree_with_brute(fn, w, u, k, v)


def test_constant_decay_is_the_constant_decay_operator():
    rng = np.random.default_rng(5)
    B, T, C = 2, 12, 4
    _, u, k, v = rand_dd(rng, B, T, C)
    wc = np.exp(rng.uniform(-3, 1.5, C))
    s0 = random_state(rng, B, C)
    for st0 in (None, s0):
        ref, rs = wkv_direct(wc, u, k, v, st0)
        wt = np.broadcast_to(wc, (B, T, C)).copy()
        for fn in (D.wkv_dd_direct, D.wkv_dd_recurrent):
            o, s = fn(wt, u, k, v, st0)
            assert normalised_error(o, ref, 1.0).max() <= 1e-13
            assert state_close(s, rs, 1e-13)


def test_hand_worked_case():
    """k = 0, v = (1, 0, 0), u = 0, rate ln 2 at step 1 (0-based): out_0 = v_0 = 1;
    out_1 = (1 + 0) / (1 + 1) = 1/2; out_2 = (1/2 * 1) / (1/2 + 1 + 1) = 1/5,
    whatever the rates of steps 0 and 2."""
    k = np.zeros((1, 3, 1))
    v = np.array([1.0, 0.0, 0.0]).reshape(1, 3, 1)
    u = np.zeros(1)
    for w0, w2 in ((0.1, 5.0), (7.0, 0.01)):
        w = np.array([w0, np.log(2.0), w2]).reshape(1, 3, 1)
        for fn in (D.wkv_dd_direct, D.wkv_dd_recurrent):
            o, _ = fn(w, u, k, v)
            np.testing.assert_allclose(o[0, :, 0], [1.0, 0.5, 0.2], rtol=1e-15, atol=0)


def test_outputs_ignore_current_and_later_rates():
    """out_t uses the state before step t's decay, so it cannot depend on w_t or
    on any later rate; from the empty state w_0 multiplies nothing either. The
    final state does depend on the last rate."""
    rng = np.random.default_rng(6)
    B, T, C = 2, 7, 3
    w, u, k, v = rand_dd(rng, B, T, C)
    o, s = D.wkv_dd_direct(w, u, k, v)
    for t in range(T):
        w2 = w.copy()
        w2[:, t:] = np.exp(rng.normal(0, 1, w2[:, t:].shape))
        o2, s2 = D.wkv_dd_direct(w2, u, k, v)
        assert np.array_equal(o2[:, :t], o[:, :t])
        assert not state_close(s2, s, 1e-6)
    w0 = w.copy()
    w0[:, 0] = 9.0
    o0, s0 = D.wkv_dd_direct(w0, u, k, v)
    assert np.array_equal(o0, o) and state_close(s0, s, 1e-15)


def test_huge_decay_wipes_the_state():
    """A rate of 1e4 at step t0 leaves only token t0 in the state after it, so
    the outputs after t0 are those of a fresh run from token t0."""
    rng = np.random.default_rng(7)
    B, T, C = 2, 12, 3
    w, u, k, v = rand_dd(rng, B, T, C)
    s0 = random_state(rng, B, C)
    t0 = 5
    w[:, t0] = 1e4
    o, s = D.wkv_dd_direct(w, u, k, v, s0)
    of, sf = D.wkv_dd_direct(w[:, t0:], u, k[:, t0:], v[:, t0:])
    assert normalised_error(o[:, t0 + 1:], of[:, 1:], 1.0).max() <= 1e-13
    assert state_close(s, sf, 1e-13)
    # and token t0's own output still sees the past
    assert normalised_error(o[:, t0], of[:, 0], 1.0).max() > 1e-3


def test_split_and_resume():
    rng = np.random.default_rng(8)
    B, T, C = 2, 15, 3
    w, u, k, v = rand_dd(rng, B, T, C)
    o, s = D.wkv_dd_recurrent(w, u, k, v)
    for cut in (1, 7, 14):
        o1, s1 = D.wkv_dd_recurrent(w[:, :cut], u, k[:, :cut], v[:, :cut])
        o2, s2 = D.wkv_dd_recurrent(w[:, cut:], u, k[:, cut:], v[:, cut:], s1)
        assert normalised_error(np.concatenate([o1, o2], axis=1), o, 1.0).max() <= 1e-13
        assert state_close(s2, s, 1e-13)


def test_steps_equal_sums_and_key_shift_invariance():
    rng = np.random.default_rng(9)
    B, T, C = 3, 14, 4
    w, u, k, v = rand_dd(rng, B, T, C, 3.0)
    s0 = random_state(rng, B, C)
    od, sd = D.wkv_dd_direct(w, u, k, v, s0)
    orr, sr = D.wkv_dd_recurrent(w, u, k, v, s0)
    assert normalised_error(orr, od, 1.0).max() <= 1e-13 and state_close(sr, sd, 1e-13)
    s0b = s0.copy()
    s0b[2] += 4.25
    ob, sb = D.wkv_dd_recurrent(w, u, k + 4.25, v, s0b)
    assert normalised_error(ob, orr, 1.0).max() <= 1e-13
    assert np.allclose(sb[2], sr[2] + 4.25, rtol=0, atol=1e-12)


def test_outputs_stay_in_the_value_range():
    rng = np.random.default_rng(10)
    B, T, C = 2, 20, 3
    w, u, k, v = rand_dd(rng, B, T, C, 4.0)
    o, _ = D.wkv_dd_recurrent(w, u, k, v)
    lo = np.minimum.accumulate(v, axis=1)
    hi = np.maximum.accumulate(v, axis=1)
    assert np.all(o >= lo - 1e-12) and np.all(o <= hi + 1e-12)


MUTANTS = [
    # past tokens decayed from their own step on
    ("exps[:, 1 + i] = k[:, i] - _decay_between(w, i + 1, t)",
     "exps[:, 1 + i] = k[:, i] - _decay_between(w, i, t)"),
    # the initial state misses step 0's decay
    ("exps[:, 0] = m0 - _decay_between(w, 0, t)", "exps[:, 0] = m0 - _decay_between(w, 1, t)"),
    # the final state misses the last step's decay
    ("exps[:, 1 + i] = k[:, i] - _decay_between(w, i + 1, T)",
     "exps[:, 1 + i] = k[:, i] - _decay_between(w, i + 1, T - 1)"),
    # half the rate in the decode step
    ("decayed = mx - w_t", "decayed = mx - 0.5 * w_t"),
]


@pytest.mark.parametrize("old,new", MUTANTS)
def test_planted_mistakes_fail_the_brute_force_pin(old, new):
    src = inspect.getsource(D)
    assert old in src
    code = src.replace(old, new).replace("from .wkv_oracle import empty_state",
                                         "from oracle.wkv_oracle import empty_state")
    ns = {"__name__": "mutant"}
    exec(compile(code, "mutant", "exec"), ns)
    rng = np.random.default_rng(12)
    w, u, k, v = rand_dd(rng, 2, 6, 2)
    s0 = random_state(rng, 2, 2)
    ok = (agree_with_brute(ns["wkv_dd_direct"], w, u, k, v, s0)
          and agree_with_brute(ns["wkv_dd_recurrent"], w, u, k, v, s0))
    assert not ok

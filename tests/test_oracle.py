"""Pins for the float64 oracle (oracle/): it is checked against things other
than itself before anything is checked against it.

* the 50-digit mpmath brute force of the defining equation (page "Linear
  attention without writing a CUDA kernel", section "The recurrence", the
  wkv_t equation) on tiny random inputs, extreme keys included;
* hand-derived closed forms at T = 1, 2, 3 and the stored worked cases under
  tests/golden/;
* invariants: outputs stay inside the range of the values mixed, a constant
  added to every key changes nothing, splitting a sequence and passing the
  state across changes nothing, the state stays canonical;
* special cases that reduce to a textbook routine: w = 0, u = 0 is a causal
  softmax mean (scipy.special.softmax); a huge w keeps only the newest past
  token; a huge |u| hands the output to the current token or to the past;
  constant keys give a geometric series.

At the end, planted mistakes (a dropped bonus, a flipped decay sign, the decay
applied one step early, the bonus leaking into the state, k and v swapped) are
run through the same pins, and each must fail at least one of them.
"""

import json
import math
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st
from scipy.special import softmax

from oracle import (
    canonical,
    empty_state,
    normalised_error,
    wkv_combine,
    wkv_direct,
    wkv_recurrent,
    wkv_segment_summary,
    wkv_step_ref,
)
from oracle.wkv_brute import wkv_brute

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_cases.json")


def rand_inputs(rng, B, T, C, kscale=1.0, wlo=0.01, whi=5.0, ustd=0.5):
    k = rng.normal(0.0, kscale, (B, T, C))
    v = rng.normal(0.0, 1.0, (B, T, C))
    w = np.exp(rng.uniform(np.log(wlo), np.log(whi), C))
    u = rng.normal(0.0, ustd, C)
    return w, u, k, v


def state_close(a, b, tol):
    """Compare two states through their canonical view (num/den and
    max_exp + ln den), which does not depend on how the state is scaled."""
    ra, La = canonical(a)
    rb, Lb = canonical(b)
    ok_r = np.all(np.abs(ra - rb) <= tol * (np.abs(rb) + 1.0))
    ok_L = np.all(np.abs(La - Lb) <= tol * np.maximum(1.0, np.abs(Lb)))
    return bool(ok_r and ok_L)


# ---------------------------------------------------------------- brute force

@settings(max_examples=25, deadline=None)
@given(seed=st.integers(0, 2**31 - 1), T=st.integers(1, 12), C=st.integers(1, 3),
       kscale=st.sampled_from([0.5, 2.0, 20.0, 60.0]))
def test_direct_and_recurrent_match_brute_force(seed, T, C, kscale):
    rng = np.random.default_rng(seed)
    w, u, k, v = rand_inputs(rng, 1, T, C, kscale=kscale)
    k = np.clip(k, -60, 60)
    ob, sb = wkv_brute(w, u, k, v)
    od, sd = wkv_direct(w, u, k, v)
    orr, sr = wkv_recurrent(w, u, k, v)
    s = 1.0
    assert normalised_error(od, ob, s).max() <= 1e-12
    assert normalised_error(orr, ob, s).max() <= 1e-12
    assert state_close(sd, sb, 1e-12)
    assert state_close(sr, sb, 1e-12)


def test_brute_force_with_initial_state():
    rng = np.random.default_rng(7)
    w, u, k, v = rand_inputs(rng, 2, 9, 3)
    s0 = np.stack([rng.normal(0, 1, (2, 3)), rng.uniform(0.5, 3.0, (2, 3)),
                   rng.normal(0, 2, (2, 3))])
    ob, sb = wkv_brute(w, u, k, v, s0)
    od, sd = wkv_direct(w, u, k, v, s0)
    orr, sr = wkv_recurrent(w, u, k, v, s0)
    assert normalised_error(od, ob, 1.0).max() <= 1e-12
    assert normalised_error(orr, ob, 1.0).max() <= 1e-12
    assert state_close(sd, sb, 1e-12) and state_close(sr, sb, 1e-12)


@pytest.mark.parametrize("kmag", [60.0, 88.0, 600.0])
def test_extreme_keys_stay_finite_and_accurate(kmag):
    rng = np.random.default_rng(11)
    T, C = 24, 4
    w, u, k, v = rand_inputs(rng, 1, T, C)
    k = rng.choice([-kmag, kmag, 0.0], size=(1, T, C))
    ob, sb = wkv_brute(w, u, k, v)
    od, sd = wkv_direct(w, u, k, v)
    orr, sr = wkv_recurrent(w, u, k, v)
    assert np.isfinite(od).all() and np.isfinite(orr).all()
    assert np.isfinite(sd).all() and np.isfinite(sr).all()
    # float64 rounding of max_exp - w grows with |max_exp|; 1e-9 bounds it at 600
    tol = 1e-12 if kmag <= 88 else 1e-9
    assert normalised_error(od, ob, 1.0).max() <= 1e-12
    assert normalised_error(orr, ob, 1.0).max() <= tol


# ------------------------------------------------------------- closed forms

def test_t1_output_is_v_and_state_is_token():
    rng = np.random.default_rng(1)
    w, u, k, v = rand_inputs(rng, 2, 1, 5)
    for fn in (wkv_direct, wkv_recurrent):
        out, s = fn(w, u, k, v)
        assert np.array_equal(out[:, 0], v[:, 0])
        np.testing.assert_allclose(s[0], v[:, 0], rtol=0, atol=0)
        np.testing.assert_allclose(s[1], 1.0, rtol=0, atol=0)
        np.testing.assert_allclose(s[2], k[:, 0], rtol=0, atol=0)


def test_t2_closed_form_and_independent_of_w():
    rng = np.random.default_rng(2)
    _, u, k, v = rand_inputs(rng, 1, 2, 4)
    expect = ((np.exp(k[0, 0]) * v[0, 0] + np.exp(u + k[0, 1]) * v[0, 1])
              / (np.exp(k[0, 0]) + np.exp(u + k[0, 1])))
    for w in (np.full(4, 0.01), np.full(4, 3.0), np.array([0.1, 1.0, 10.0, 100.0])):
        for fn in (wkv_direct, wkv_recurrent):
            out, _ = fn(w, u, k, v)
            np.testing.assert_allclose(out[0, 1], expect, rtol=1e-14, atol=0)


def test_t3_closed_form():
    w, u = 0.7, 0.3
    k = [0.5, -1.0, 2.0]
    v = [1.0, -2.0, 3.0]
    num = math.exp(-w + k[0]) * v[0] + math.exp(k[1]) * v[1] + math.exp(u + k[2]) * v[2]
    den = math.exp(-w + k[0]) + math.exp(k[1]) + math.exp(u + k[2])
    for fn in (wkv_direct, wkv_recurrent):
        out, _ = fn([w], [u], np.reshape(k, (1, 3, 1)), np.reshape(v, (1, 3, 1)))
        assert out[0, 0, 0] == 1.0
        assert abs(out[0, 2, 0] - num / den) <= 1e-15 * abs(num / den)


def test_stored_worked_cases():
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    assert len(cases) >= 3
    for cs in cases:
        args = (np.array(cs["w"]), np.array(cs["u"]), np.array(cs["k"]), np.array(cs["v"]),
                None if cs["state_in"] is None else np.array(cs["state_in"]))
        for fn in (wkv_direct, wkv_recurrent):
            out, s = fn(*args)
            np.testing.assert_allclose(out, np.array(cs["out"]), rtol=1e-13, atol=1e-15)
            assert state_close(s, np.array(cs["state_out"]), 1e-13)


def test_geometric_closed_form():
    # k = 0, u = 0: the denominator before the bonus is 1 + e^-w + ... + e^-(t-2)w
    # for t >= 2 (1-based), so the bonus weight 1 shares with it.
    T, C = 40, 3
    w = np.array([0.05, 0.7, 4.0])
    u = np.zeros(C)
    k = np.zeros((1, T, C))
    v = np.random.default_rng(3).normal(size=(1, T, C))
    out, s = wkv_recurrent(w, u, k, v)
    for c in range(C):
        for t in range(T):  # 0-based t: past tokens i < t with decay (t-1-i) w
            weights = np.array([math.exp(-(t - 1 - i) * w[c]) for i in range(t)] + [1.0])
            vals = np.concatenate([v[0, :t, c], [v[0, t, c]]])
            assert abs(out[0, t, c] - (weights @ vals) / weights.sum()) <= 1e-13
    D = 1.0 + sum(math.exp(-j * w[0]) for j in range(1, T))
    _, L = canonical(s)
    assert abs(L[0, 0] - math.log(D)) <= 1e-13
    # constant values give a constant output
    out_c, _ = wkv_direct(w, u, k, np.full((1, T, C), 2.5))
    np.testing.assert_allclose(out_c, 2.5, rtol=1e-15)


# ----------------------------------------------------------------- invariants

@settings(max_examples=20, deadline=None)
@given(seed=st.integers(0, 2**31 - 1), T=st.integers(1, 40))
def test_output_inside_range_of_mixed_values(seed, T):
    rng = np.random.default_rng(seed)
    w, u, k, v = rand_inputs(rng, 2, T, 3, kscale=3.0)
    s0 = np.stack([rng.normal(0, 1, (2, 3)), rng.uniform(0.5, 2.0, (2, 3)),
                   rng.normal(0, 1, (2, 3))])
    out, _ = wkv_recurrent(w, u, k, v, s0)
    r0 = s0[0] / s0[1]
    for t in range(T):
        lo = np.minimum(v[:, : t + 1].min(axis=1), r0)
        hi = np.maximum(v[:, : t + 1].max(axis=1), r0)
        assert np.all(out[:, t] >= lo - 1e-12) and np.all(out[:, t] <= hi + 1e-12)


@settings(max_examples=20, deadline=None)
@given(seed=st.integers(0, 2**31 - 1), shift=st.floats(-30, 30))
def test_key_shift_invariance(seed, shift):
    rng = np.random.default_rng(seed)
    w, u, k, v = rand_inputs(rng, 1, 20, 3)
    o1, s1 = wkv_recurrent(w, u, k, v)
    o2, s2 = wkv_recurrent(w, u, k + shift, v)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s2[:2], s1[:2], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s2[2], s1[2] + shift, rtol=1e-12, atol=1e-11)
    od, _ = wkv_direct(w, u, k + shift, v)
    np.testing.assert_allclose(od, o1, rtol=1e-12, atol=1e-12)


def test_split_resume_and_step_equivalence():
    rng = np.random.default_rng(4)
    w, u, k, v = rand_inputs(rng, 2, 30, 4)
    full, sf = wkv_direct(w, u, k, v)
    for cut in (1, 13, 29):
        o1, s1 = wkv_direct(w, u, k[:, :cut], v[:, :cut])
        o2, s2 = wkv_direct(w, u, k[:, cut:], v[:, cut:], s1)
        np.testing.assert_allclose(np.concatenate([o1, o2], axis=1), full, rtol=1e-12, atol=1e-13)
        assert state_close(s2, sf, 1e-12)
    state = empty_state(2, 4)
    for t in range(30):
        o, state = wkv_step_ref(w, u, k[:, t], v[:, t], state)
        np.testing.assert_allclose(o, full[:, t], rtol=1e-12, atol=1e-13)
    assert state_close(state, sf, 1e-12)


def test_segment_combine_is_associative_and_matches_sequence():
    rng = np.random.default_rng(5)
    w, u, k, v = rand_inputs(rng, 2, 24, 3, kscale=4.0)
    cuts = [0, 5, 6, 17, 24]
    segs = [wkv_segment_summary(w, k[:, a:b], v[:, a:b]) for a, b in zip(cuts, cuts[1:])]
    lens = [b - a for a, b in zip(cuts, cuts[1:])]
    s0 = np.stack([rng.normal(0, 1, (2, 3)), rng.uniform(0.5, 2.0, (2, 3)), rng.normal(0, 1, (2, 3))])
    left = s0
    for sg, L in zip(segs, lens):
        left = wkv_combine(left, sg, L, w)
    _, want = wkv_direct(w, u, k, v, s0)
    assert state_close(left, want, 1e-12)
    # ((s0 . A) . B) == s0 . (A . B): fold the last two segments first
    bc = wkv_combine(segs[2], segs[3], lens[3], w)
    right = wkv_combine(wkv_combine(wkv_combine(s0, segs[0], lens[0], w), segs[1], lens[1], w),
                        bc, lens[2] + lens[3], w)
    assert state_close(right, want, 1e-12)
    # the empty state is the identity on both sides
    e = empty_state(2, 3)
    assert state_close(wkv_combine(e, segs[1], lens[1], w), segs[1], 0)
    assert state_close(wkv_combine(segs[1], e, 0, w), segs[1], 0)


def test_state_is_canonical():
    rng = np.random.default_rng(6)
    w, u, k, v = rand_inputs(rng, 3, 50, 5, kscale=5.0)
    for t in (1, 2, 17, 50):
        for fn in (wkv_direct, wkv_recurrent):
            _, s = fn(w, u, k[:, :t], v[:, :t])
            n, d, _m = s
            assert np.all(d >= 1.0 - 1e-15) and np.all(d <= t + 1e-12)
            assert np.all(np.abs(n) <= d * np.abs(v[:, :t]).max(axis=1) + 1e-12)


def test_empty_sequence_and_empty_state():
    rng = np.random.default_rng(8)
    w, u, k, v = rand_inputs(rng, 2, 0, 3)
    for fn in (wkv_direct, wkv_recurrent):
        out, s = fn(w, u, k, v)
        assert out.shape == (2, 0, 3)
        np.testing.assert_array_equal(s, empty_state(2, 3))


# -------------------------------------------------------------- special cases

def test_zero_decay_zero_bonus_is_causal_softmax_mean():
    rng = np.random.default_rng(9)
    T, C = 25, 3
    k = rng.normal(0, 2.0, (1, T, C))
    v = rng.normal(0, 1.0, (1, T, C))
    out, _ = wkv_direct(np.zeros(C), np.zeros(C), k, v)
    out_r, _ = wkv_recurrent(np.zeros(C), np.zeros(C), k, v)
    for c in range(C):
        for t in range(T):
            want = softmax(k[0, : t + 1, c]) @ v[0, : t + 1, c]
            assert abs(out[0, t, c] - want) <= 1e-13
            assert abs(out_r[0, t, c] - want) <= 1e-13


def test_huge_decay_keeps_only_newest_past_token():
    rng = np.random.default_rng(10)
    T, C = 12, 3
    k = rng.normal(0, 1.0, (1, T, C))
    v = rng.normal(0, 1.0, (1, T, C))
    u = rng.normal(0, 0.5, C)
    w = np.full(C, 1e4)
    for fn in (wkv_direct, wkv_recurrent):
        out, _ = fn(w, u, k, v)
        for t in range(1, T):
            p = softmax(np.stack([k[0, t - 1], u + k[0, t]]), axis=0)
            want = p[0] * v[0, t - 1] + p[1] * v[0, t]
            np.testing.assert_allclose(out[0, t], want, rtol=1e-13, atol=1e-14)


def test_huge_bonus_either_sign():
    rng = np.random.default_rng(12)
    T, C = 10, 2
    k = rng.normal(0, 1.0, (1, T, C))
    v = rng.normal(0, 1.0, (1, T, C))
    w = np.array([0.3, 2.0])
    for fn in (wkv_direct, wkv_recurrent):
        out, _ = fn(w, np.full(C, 1e3), k, v)
        np.testing.assert_array_equal(out, v)
        out_neg, _ = fn(w, np.full(C, -1e3), k, v)
        past_only, _ = fn(w, np.full(C, -1e3), k, v)
        assert np.array_equal(out_neg[0, 0], v[0, 0])
        for t in range(1, T):
            for c in range(C):
                wt = np.exp(k[0, :t, c] - (t - 1 - np.arange(t)) * w[c])
                want = wt @ v[0, :t, c] / wt.sum()
                assert abs(past_only[0, t, c] - want) <= 1e-13


# ----------------------------------------------------- planted mistakes fail

def _mutant(kind):
    """A copy of the recurrence with one plausible mistake planted in it."""

    def run(w, u, k, v, state_in=None):
        w, u = np.asarray(w, float), np.asarray(u, float)
        k, v = np.asarray(k, float), np.asarray(v, float)
        B, T, C = k.shape
        n, d, m = empty_state(B, C) if state_in is None else np.asarray(state_in, float).copy()
        out = np.empty((B, T, C))
        for t in range(T):
            kt, vt = k[:, t], v[:, t]
            if kind == "swap_kv":
                kt, vt = vt, kt
            bonus = 0.0 if kind == "drop_bonus" else u
            cur = bonus + kt
            mm = m - w if kind == "decay_early" else m
            ref = np.maximum(mm, cur)
            a, b = np.exp(mm - ref), np.exp(cur - ref)
            out[:, t] = (a * n + b * vt) / (a * d + b)
            dec = m + w if kind == "decay_sign" else m - w
            newk = kt + u if kind == "bonus_in_state" else kt
            ref2 = np.maximum(dec, newk)
            a2, b2 = np.exp(dec - ref2), np.exp(newk - ref2)
            n, d, m = a2 * n + b2 * vt, a2 * d + b2, ref2
        return out, np.stack([n, d, m])

    return run


def _pins_failed(fn):
    """Run a handful of pins against fn; return the names of those that fail."""
    failed = []
    rng = np.random.default_rng(21)
    w, u, k, v = rand_inputs(rng, 1, 6, 3)
    ob, sb = wkv_brute(w, u, k, v)
    o, s = fn(w, u, k, v)
    if normalised_error(o, ob, 1.0).max() > 1e-12 or not state_close(s, sb, 1e-12):
        failed.append("brute")
    with open(GOLDEN) as f:
        cs = json.load(f)["cases"][0]
    o, _ = fn(np.array(cs["w"]), np.array(cs["u"]), np.array(cs["k"]), np.array(cs["v"]))
    if not np.allclose(o, np.array(cs["out"]), rtol=1e-13, atol=1e-15):
        failed.append("t3")
    kk = rng.normal(0, 2.0, (1, 8, 2))
    vv = rng.normal(0, 1.0, (1, 8, 2))
    o, _ = fn(np.zeros(2), np.zeros(2), kk, vv)
    want = np.array([[softmax(kk[0, : t + 1, c]) @ vv[0, : t + 1, c] for c in range(2)]
                     for t in range(8)])
    if not np.allclose(o[0], want, rtol=1e-12, atol=1e-13):
        failed.append("softmax")
    return failed


def test_oracle_passes_the_mutation_pins():
    assert _pins_failed(wkv_recurrent) == []
    assert _pins_failed(wkv_direct) == []


@pytest.mark.parametrize("kind", ["drop_bonus", "decay_sign", "decay_early",
                                  "bonus_in_state", "swap_kv"])
def test_planted_mistake_is_caught(kind):
    assert _pins_failed(_mutant(kind)), f"planted mistake {kind!r} slipped through every pin"

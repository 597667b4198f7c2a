"""Pins of the token-shift oracle (oracle/wkv_shift.py) against what the
definition fixes without restating it: the mixing fraction's end points
(identity and exact one-token shift), its midpoint, affinity in mu,
split/resume and one-token steps, constant sequences, and a hand-worked case
of the page's equations (page "RWKV-v6 Architecture: Attention-Free Linear
Transformers", section "The Core Components of the RWKV-v6 Time-Mixing
Block", item 1 "Data-Dependent Token Shift (DD-LERP)"). Each pin fails for a
plausible mistake: a flipped sign, the wrong neighbour (t + 1), a mixed-up
projection index, or a lost carry across calls."""

import numpy as np
import pytest

from oracle.wkv_shift import token_shift


def _case(seed, B=2, T=7, C=5, P=3):
    g = np.random.default_rng(seed)
    return g.normal(size=(B, T, C)), g.uniform(0, 1, (P, C)), g.normal(size=(B, C))


def test_zero_fraction_is_the_identity(fn=token_shift):
    x, _, xp = _case(1)
    mix, last = fn(x, np.zeros((2, 5)), xp)
    assert np.array_equal(mix[0], x) and np.array_equal(mix[1], x)
    assert np.array_equal(last, x[:, -1])


def test_unit_fraction_is_the_previous_token(fn=token_shift):
    # x + (x_prev - x) * 1 rounds twice in float64: within 2 ulp of the larger
    # of the two operands
    x, _, xp = _case(2)
    mix, _ = fn(x, np.ones((1, 5)), xp)
    before = np.concatenate([xp[:, None], x[:, :-1]], axis=1)
    bound = 4 * np.finfo(np.float64).eps * np.maximum(np.abs(before), np.abs(x))
    assert np.all(np.abs(mix[0] - before) <= bound)


def test_missing_previous_token_is_zero(fn=token_shift):
    x, mu, _ = _case(3)
    a, _ = fn(x, mu, None)
    b, _ = fn(x, mu, np.zeros((2, 5)))
    assert np.array_equal(a, b)
    assert np.allclose(a[:, :, 0], x[None, :, 0] * (1 - mu[:, None, :]), rtol=0, atol=1e-15)


def test_half_fraction_is_the_midpoint(fn=token_shift):
    x, _, xp = _case(4)
    mix, _ = fn(x, np.full((1, 5), 0.5), xp)
    before = np.concatenate([xp[:, None], x[:, :-1]], axis=1)
    np.testing.assert_allclose(mix[0], (before + x) / 2, rtol=1e-15, atol=1e-15)


def test_affine_in_the_fraction(fn=token_shift):
    x, _, xp = _case(5)
    g = np.random.default_rng(6)
    m1, m2 = g.uniform(0, 1, (1, 5)), g.uniform(0, 1, (1, 5))
    a = 0.3
    lhs, _ = fn(x, a * m1 + (1 - a) * m2, xp)
    r1, _ = fn(x, m1, xp)
    r2, _ = fn(x, m2, xp)
    np.testing.assert_allclose(lhs, a * r1 + (1 - a) * r2, rtol=1e-13, atol=1e-14)


def test_projections_use_their_own_fraction(fn=token_shift):
    x, mu, xp = _case(7, P=4)
    mix, _ = fn(x, mu, xp)
    for p in range(4):
        one, _ = fn(x, mu[p:p + 1], xp)
        assert np.array_equal(mix[p], one[0])


@pytest.mark.parametrize("cut", [0, 1, 3, 7])
def test_split_and_resume(cut, fn=token_shift):
    x, mu, xp = _case(8)
    full, last = fn(x, mu, xp)
    a, la = fn(x[:, :cut], mu, xp)
    b, lb = fn(x[:, cut:], mu, la)
    assert np.array_equal(np.concatenate([a, b], axis=2), full)
    assert np.array_equal(lb, last)


def test_one_token_steps_match_the_sequence(fn=token_shift):
    x, mu, xp = _case(9)
    full, _ = fn(x, mu, xp)
    prev = xp
    for t in range(x.shape[1]):
        step, prev = fn(x[:, t:t + 1], mu, prev)
        assert np.array_equal(step[:, :, 0], full[:, :, t])


def test_constant_sequence_is_unchanged(fn=token_shift):
    g = np.random.default_rng(10)
    c = g.normal(size=(2, 1, 5))
    x = np.repeat(c, 9, axis=1)
    mix, _ = fn(x, g.uniform(0, 1, (3, 5)), c[:, 0])
    np.testing.assert_allclose(mix, np.broadcast_to(x, mix.shape), rtol=1e-15, atol=1e-15)


def test_hand_worked_case(fn=token_shift):
    # B = 1, T = 2, C = 2, no previous token (zeros); two projections with
    # mu_0 = (0.25, 1) and mu_1 = (0, 0.5). By x' = x_t + (x_{t-1} - x_t) mu:
    #   t = 0, x = (1, 2),  x_{-1} = (0, 0):
    #     p0: (1 - 0.25, 2 - 2) = (0.75, 0)      p1: (1, 2 - 1) = (1, 1)
    #   t = 1, x = (3, 5),  x_0 = (1, 2):
    #     p0: (3 - 2 * 0.25, 5 - 3) = (2.5, 2)   p1: (3, 5 - 1.5) = (3, 3.5)
    x = np.array([[[1.0, 2.0], [3.0, 5.0]]])
    mu = np.array([[0.25, 1.0], [0.0, 0.5]])
    mix, last = fn(x, mu)
    expect = np.array([[[[0.75, 0.0], [2.5, 2.0]]], [[[1.0, 1.0], [3.0, 3.5]]]])
    assert np.array_equal(mix, expect)
    assert np.array_equal(last, [[3.0, 5.0]])


def test_empty_sequence_passes_the_previous_token_on(fn=token_shift):
    _, mu, xp = _case(11)
    mix, last = fn(np.zeros((2, 0, 5)), mu, xp)
    assert mix.shape == (3, 2, 0, 5)
    assert np.array_equal(last, xp)


def _planted(kind):
    def f(x, mu, x_prev=None):
        x = np.asarray(x, np.float64)
        B, T, C = x.shape
        prev = np.zeros((B, C)) if x_prev is None else np.asarray(x_prev, np.float64)
        if kind == "next":  # the following token instead of the previous one
            nb = np.concatenate([x[:, 1:], x[:, -1:]], axis=1)
        else:
            nb = np.concatenate([prev[:, None], x[:, :-1]], axis=1)
        sgn = -1.0 if kind == "sign" else 1.0
        m = mu[::-1] if kind == "index" else mu
        out = x[None] + sgn * (nb - x)[None] * np.asarray(m)[:, None, None, :]
        return out, (prev if kind == "carry" else x[:, -1])
    return f


@pytest.mark.parametrize("kind", ["next", "sign", "index", "carry"])
def test_planted_mistakes_are_caught(kind):
    """The pins above, run against a deliberately wrong variant, must fail
    for at least one of them."""
    bad = _planted(kind)
    pins = [test_unit_fraction_is_the_previous_token, test_hand_worked_case,
            test_projections_use_their_own_fraction, test_one_token_steps_match_the_sequence,
            test_constant_sequence_is_unchanged, test_missing_previous_token_is_zero]
    failed = 0
    for pin in pins:
        try:
            pin(fn=bad)
        except AssertionError:
            failed += 1
    for cut in (1, 3):
        try:
            test_split_and_resume(cut, fn=bad)
        except AssertionError:
            failed += 1
    assert failed > 0, f"no pin catches the planted mistake '{kind}'"

"""Float64 CPU oracle for the RWKV weighted-key-value (WKV) operator.

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module. It shares no code with the HIP library
and imports nothing from it: inputs come in as numpy arrays and results go out as
numpy arrays.

What is computed
----------------
Source: the page "Linear attention without writing a CUDA kernel", section
"The recurrence".

* Its displayed equation defines, per channel, the output at position t as a
  ratio of two sums over the past tokens i < t: each past token carries the
  weight exp(k_i - (t-1-i) w), so the newest past token is not decayed at all
  and every further step back costs one more factor exp(-w); the current token
  enters both sums with the bonus weight exp(u + k_t). The numerator weights
  v_i, the denominator weights 1.
* The same section's code carries the state as three arrays shaped like k:
  numerator, denominator and a running maximum exponent, rescaled the way a
  stable softmax is, so that every step costs the same. The output of a step
  uses the state as it stands plus the bonus term; only afterwards is the state
  decayed by w and the current token (without u) added.

Conventions fixed here (the pages leave them open; every one is listed in the
design notes):

* Shapes: k, v, out are (B, T, C); w, u are (C,); a state is (3, B, C) holding
  the planes num, den, max_exp. Positions are 0-based in code, so the page's
  "t-1-i" becomes "t-1-i" with t, i both 0-based (the same difference).
* A non-empty initial state (n0, d0, m0) is the summary of tokens that came
  before position 0: it contributes n0 * exp(m0 - t w) to the numerator at
  position t (it has been decayed once per token consumed since), d0 likewise.
* The empty state is (0, 0, -1e38): finite, never -inf, so that differences of
  two empty exponents stay 0 rather than NaN.
* The state after the last token is inclusive of it: the next step's output
  uses it undecayed, exactly as the page's step function returns it.

Every function works in float64 on copies of its inputs.
"""

from __future__ import annotations

import numpy as np

# Exponent of the empty state. Finite on purpose (see module docstring).
EMPTY_MAX_EXP = -1.0e38


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def empty_state(B: int, C: int) -> np.ndarray:
    """The state before any token: num = den = 0, max_exp = -1e38."""
    s = np.zeros((3, B, C), dtype=np.float64)
    s[2] = EMPTY_MAX_EXP
    return s


def _check(w, u, k, v, state_in):
    w, u, k, v = _f64(w), _f64(u), _f64(k), _f64(v)
    if k.ndim != 3 or v.shape != k.shape:
        raise ValueError(f"k and v must both be (B, T, C); got {k.shape} and {v.shape}")
    B, T, C = k.shape
    if w.shape != (C,) or u.shape != (C,):
        raise ValueError(f"w and u must be ({C},); got {w.shape} and {u.shape}")
    if state_in is None:
        state_in = empty_state(B, C)
    state_in = _f64(state_in)
    if state_in.shape != (3, B, C):
        raise ValueError(f"state must be (3, {B}, {C}); got {state_in.shape}")
    return w, u, k, v, state_in.copy()


# ---------------------------------------------------------------------------
# O1: the definition, written out as a sum (O(T^2) per lane; small inputs only).
# ---------------------------------------------------------------------------

def _ratio_of_sums(exps, num_coef, den_coef):
    """sum(num_coef * e^exps) / sum(den_coef * e^exps) along axis 1, with the
    largest exponent factored out first (it cancels between the two sums)."""
    top = exps.max(axis=1, keepdims=True)
    e = np.exp(exps - top)
    return (num_coef * e).sum(axis=1) / (den_coef * e).sum(axis=1)


def wkv_direct(w, u, k, v, state_in=None):
    """WKV by its defining equation (page "Linear attention without writing a
    CUDA kernel", section "The recurrence", the wkv_t equation), extended to a
    non-empty initial state as described in the module docstring.

    For every position t the full list of terms is built and summed; nothing is
    carried from one position to the next. Returns (out, state_out) with out of
    shape (B, T, C) and state_out = (N e^-M, D e^-M, M) of shape (3, B, C), where
    M is the largest exponent among the terms left after the last token.
    """
    w, u, k, v, s0 = _check(w, u, k, v, state_in)
    B, T, C = k.shape
    n0, d0, m0 = s0
    out = np.empty((B, T, C), dtype=np.float64)
    for t in range(T):
        # term 0: the initial state, decayed once per token consumed so far.
        # terms 1..t: past tokens i < t, newest undecayed.
        # term t+1: the current token with the bonus u.
        exps = np.empty((B, t + 2, C), dtype=np.float64)
        numc = np.empty_like(exps)
        denc = np.empty_like(exps)
        exps[:, 0] = m0 - t * w
        numc[:, 0] = n0
        denc[:, 0] = d0
        if t > 0:
            age = (t - 1 - np.arange(t, dtype=np.float64))[None, :, None]
            exps[:, 1:t + 1] = k[:, :t] - age * w
            numc[:, 1:t + 1] = v[:, :t]
            denc[:, 1:t + 1] = 1.0
        exps[:, t + 1] = u + k[:, t]
        numc[:, t + 1] = v[:, t]
        denc[:, t + 1] = 1.0
        out[:, t] = _ratio_of_sums(exps, numc, denc)
    state_out = _summary_by_definition(w, k, v, n0, d0, m0)
    return out, state_out


def _summary_by_definition(w, k, v, n0, d0, m0):
    """Inclusive state after all T tokens, by the sum: token i has been decayed
    T-1-i times, the initial state T times; no bonus term."""
    B, T, C = k.shape
    exps = np.empty((B, T + 1, C), dtype=np.float64)
    numc = np.empty_like(exps)
    denc = np.empty_like(exps)
    exps[:, 0] = m0 - T * w
    numc[:, 0] = n0
    denc[:, 0] = d0
    if T > 0:
        age = (T - 1 - np.arange(T, dtype=np.float64))[None, :, None]
        exps[:, 1:] = k - age * w
        numc[:, 1:] = v
        denc[:, 1:] = 1.0
    top = exps.max(axis=1)
    e = np.exp(exps - top[:, None])
    N = (numc * e).sum(axis=1)
    D = (denc * e).sum(axis=1)
    return np.stack([N, D, top])


# ---------------------------------------------------------------------------
# O2: the stabilised recurrence (one step per token, vectorised over lanes).
# ---------------------------------------------------------------------------

def _share(x):
    """1 / (1 + e^-x) for x in [-inf, inf]: e^-x may overflow to inf for very
    negative x, which gives the correct limit 0 (the warning is silenced)."""
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def _log_add(a, b):
    """log(e^a + e^b) = max(a, b) + log(1 + e^-|a - b|), for a or b = -inf too
    (not both)."""
    return np.maximum(a, b) + np.log1p(np.exp(-np.abs(a - b)))


def wkv_step_ref(w, u, k_t, v_t, state):
    """One decode step, from the sum definition (page "Linear attention
    without writing a CUDA kernel", section "The recurrence", the wkv_t
    equation and its running-state form).

    k_t, v_t: (B, C) for one position; state: (3, B, C). Returns (out_t, new
    state).

    Written as a running weighted mean rather than as rescaled sums: the state
    (num, den, max_exp) stands for the sums N = num e^max_exp and
    D = den e^max_exp, so it is read as two numbers per lane, the total weight
    of the past as its logarithm, log D = max_exp + ln den, and the mean of the
    past values under those weights, r = N / D = num / den (an empty state has
    log D = -inf). The output at this position is then the mean of two groups,
    the past (weight D, mean r) and the current token (weight e^(u + k_t),
    value v_t); the past's share of the total is
    D / (D + e^(u + k_t)) = 1 / (1 + e^-(log D - u - k_t)). After the output
    the past weight decays by e^-w and the token joins it at weight e^(k_t),
    without the bonus: log D' = log(e^(log D - w) + e^(k_t)), and r' is again
    a two-group mean with the past's share taken at exponents log D - w and
    k_t. The new state is handed back as (num, den, max_exp) = (r', 1, log D'),
    which stands for the same two sums.
    """
    w, u = _f64(w), _f64(u)
    k_t, v_t = _f64(k_t), _f64(v_t)
    num, den, mx = (_f64(p) for p in state)
    with np.errstate(divide="ignore", invalid="ignore"):
        filled = den > 0
        log_d = np.where(filled, mx + np.log(np.where(filled, den, 1.0)), -np.inf)
        mean = np.where(filled, num / np.where(filled, den, 1.0), 0.0)

    # output: past (weight D) against the current token (weight e^(u + k_t))
    gap = log_d - (u + k_t)
    out_t = _share(gap) * mean + _share(-gap) * v_t

    # the past decays by one step, the token joins without the bonus
    gap2 = (log_d - w) - k_t
    new_mean = _share(gap2) * mean + _share(-gap2) * v_t
    new_log_d = _log_add(log_d - w, k_t)
    return out_t, np.stack([new_mean, np.ones_like(new_mean), new_log_d])


def wkv_recurrent(w, u, k, v, state_in=None):
    """WKV over a whole (B, T, C) sequence by T successive decode steps
    (wkv_step_ref). Returns (out, state_out) like wkv_direct."""
    w, u, k, v, state = _check(w, u, k, v, state_in)
    B, T, C = k.shape
    out = np.empty((B, T, C), dtype=np.float64)
    for t in range(T):
        out[:, t], state = wkv_step_ref(w, u, k[:, t], v[:, t], state)
    return out, state


# ---------------------------------------------------------------------------
# The receptance gate on the output.
# ---------------------------------------------------------------------------
# The page "RWKV-v6 Architecture: Attention-Free Linear Transformers" gates
# its recurrence's output elementwise with sigmoid(r_t) (the output equation
# of its recurrence), and the page "RWKV: Merging Transformer Training with
# RNN Speed" (Time-Mixing block) describes the receptance as the gate that
# decides how much of the accumulated history passes on. Applied to this
# operator's output: out_t = sigmoid(r_t) * wkv_t per channel.

def sigmoid(x):
    """The logistic function 1 / (1 + e^-x), evaluated without overflow."""
    x = _f64(x)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    e = np.exp(x[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def wkv_gated(w, u, k, v, r, state_in=None):
    """(sigmoid(r) * wkv, state_out), wkv from the defining equation
    (wkv_direct); r has k's shape. The state is the ungated one."""
    out, st = wkv_direct(w, u, k, v, state_in)
    return sigmoid(r) * out, st


# ---------------------------------------------------------------------------
# Segment summaries and their composition (the time-parallel form).
# ---------------------------------------------------------------------------
# The page "RWKV-v6 Architecture: Attention-Free Linear Transformers", section
# on architectural duality, and the page "RWKV: Merging Transformer Training
# with RNN Speed", paragraph on the time-parallel mode, state that the same
# computation can run as an associative prefix scan over time. For this
# operator the composition follows from the sum definition: a segment of L
# tokens maps a state S (decayed L times while it passes) to
# S e^{-L w} + (the segment's own state from empty).

def wkv_segment_summary(w, k, v):
    """State after running the segment k, v (B, L, C) from the empty state:
    (N, D, M) with M the largest exponent; the summary's length is k.shape[1]."""
    w, k, v = _f64(w), _f64(k), _f64(v)
    B, L, C = k.shape
    z = np.zeros((B, C))
    return _summary_by_definition(w, k, v, z, z, np.full((B, C), EMPTY_MAX_EXP))


def wkv_combine(first, second, second_len, w):
    """Compose two adjacent segment states: `first` (any state, as (3, B, C))
    followed by `second` (the summary of a segment of `second_len` tokens
    started from empty). The first is decayed by second_len * w while the
    second segment passes, then the two sums are added, relative to the larger
    exponent."""
    w = _f64(w)
    n1, d1, m1 = (_f64(p) for p in first)
    n2, d2, m2 = (_f64(p) for p in second)
    a = m1 - second_len * w
    top = np.maximum(a, m2)
    f1 = np.exp(a - top)
    f2 = np.exp(m2 - top)
    return np.stack([f1 * n1 + f2 * n2, f1 * d1 + f2 * d2, top])


# ---------------------------------------------------------------------------
# Comparison helpers.
# ---------------------------------------------------------------------------

def canonical(state):
    """Representation-free view of a state: (r, L) with r = num/den (the value a
    following output would tend to with no new weight) and L = max_exp + ln(den)
    (the log of the true denominator sum). (n, d, m) and (n e^x, d e^x, m - x)
    describe the same state and give the same (r, L). Lanes with den = 0 give
    r = 0, L = -inf."""
    n, d, m = (_f64(p) for p in state)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(d > 0, n / np.where(d > 0, d, 1.0), 0.0)
        L = np.where(d > 0, m + np.log(np.where(d > 0, d, 1.0)), -np.inf)
    return r, L


def normalised_error(got, ref, scale):
    """Elementwise |got - ref| / (|ref| + scale). `scale` is the RMS of v over
    the tensor, so that outputs near zero (they are convex mixes of v and cross
    zero) are judged against the size of the data rather than against 0."""
    got = _f64(got)
    ref = _f64(ref)
    return np.abs(got - ref) / (np.abs(ref) + scale)

"""Arbitrary-precision brute force for the WKV operator (mpmath, 50 digits).

TEST INFRASTRUCTURE, like the rest of this package: it is the yardstick for the
float64 oracle on tiny inputs, and nothing on the HIP side uses it.

It evaluates the defining equation of the page "Linear attention without
writing a CUDA kernel", section "The recurrence" (the wkv_t equation), term by
term with mpmath's exp. mpmath's exponent range is unbounded for practical
purposes, so no maximum is factored out: the sums are formed exactly as written.
A non-empty initial state (n0, d0, m0) contributes n0 * exp(m0 - t w) and
d0 * exp(m0 - t w) at 0-based position t (the reading stated in the float64
oracle's docstring).
"""

from __future__ import annotations

import mpmath
import numpy as np


def wkv_brute(w, u, k, v, state_in=None, dps: int = 50):
    """Returns (out, state_out) as float64 arrays rounded from mpmath values.

    out: (B, T, C). state_out: (3, B, C) as (N e^-M, D e^-M, M), M the largest
    exponent present after the last token (the initial state's exponent counts
    only if its den is non-zero).
    """
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    B, T, C = k.shape
    if state_in is None:
        n0 = np.zeros((B, C))
        d0 = np.zeros((B, C))
        m0 = np.full((B, C), -1e38)
    else:
        n0, d0, m0 = (np.asarray(p, dtype=np.float64) for p in state_in)
    out = np.empty((B, T, C))
    state = np.empty((3, B, C))
    with mpmath.workdps(dps):
        mpf, exp = mpmath.mpf, mpmath.exp
        for b in range(B):
            for c in range(C):
                wc, uc = mpf(w[c]), mpf(u[c])
                ks = [mpf(x) for x in k[b, :, c]]
                vs = [mpf(x) for x in v[b, :, c]]
                has_state = d0[b, c] != 0.0 or n0[b, c] != 0.0
                for t in range(T):
                    num = mpf(0)
                    den = mpf(0)
                    if has_state:
                        f = exp(mpf(m0[b, c]) - t * wc)
                        num += mpf(n0[b, c]) * f
                        den += mpf(d0[b, c]) * f
                    for i in range(t):
                        f = exp(ks[i] - (t - 1 - i) * wc)
                        num += f * vs[i]
                        den += f
                    f = exp(uc + ks[t])
                    num += f * vs[t]
                    den += f
                    out[b, t, c] = float(num / den)
                # inclusive state after the last token
                terms = []
                if has_state:
                    terms.append((mpf(m0[b, c]) - T * wc, mpf(n0[b, c]), mpf(d0[b, c])))
                for i in range(T):
                    terms.append((ks[i] - (T - 1 - i) * wc, vs[i], mpf(1)))
                live = [x for x in terms if x[2] != 0]
                if not live:
                    state[:, b, c] = (0.0, 0.0, -1e38)
                    continue
                top = max(x[0] for x in live)
                N = sum((nc * exp(e - top) for e, nc, _ in terms), mpf(0))
                D = sum((dc * exp(e - top) for e, _, dc in terms), mpf(0))
                state[:, b, c] = (float(N), float(D), float(top))
    return out, state


def wkv_dd_brute(w, u, k, v, state_in=None, dps: int = 50):
    """The per-token-decay operator (oracle/wkv_decay.py) in 50-digit mpmath,
    written as a linear recurrence on the raw sums rather than as a sum over
    tokens: before step t the numerator and denominator sums are multiplied by
    the factor exp(-w_t) and the token is added with weight exp(k_t); the
    output of step t is formed from the sums before that multiplication plus
    the current token at exp(u + k_t). No maximum is factored out (mpmath's
    exponent range makes that unnecessary).

    Returns (out, state_out) rounded to float64, state_out as
    (N e^-M, D e^-M, M) with M the largest exponent among the terms present,
    tracked alongside the sums."""
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    B, T, C = k.shape
    if state_in is None:
        n0, d0, m0 = np.zeros((B, C)), np.zeros((B, C)), np.full((B, C), -1e38)
    else:
        n0, d0, m0 = (np.asarray(p, dtype=np.float64) for p in state_in)
    out = np.empty((B, T, C))
    state = np.empty((3, B, C))
    with mpmath.workdps(dps):
        mpf, exp = mpmath.mpf, mpmath.exp
        for b in range(B):
            for c in range(C):
                has_state = d0[b, c] != 0.0 or n0[b, c] != 0.0
                if has_state:
                    N = mpf(n0[b, c]) * exp(mpf(m0[b, c]))
                    D = mpf(d0[b, c]) * exp(mpf(m0[b, c]))
                    top = mpf(m0[b, c])
                else:
                    N, D, top = mpf(0), mpf(0), None
                uc = mpf(u[c])
                for t in range(T):
                    kt, vt = mpf(k[b, t, c]), mpf(v[b, t, c])
                    f = exp(uc + kt)
                    out[b, t, c] = float((N + f * vt) / (D + f))
                    decay = exp(-mpf(w[b, t, c]))
                    g = exp(kt)
                    N = N * decay + g * vt
                    D = D * decay + g
                    top = kt if top is None else max(top - mpf(w[b, t, c]), kt)
                if top is None:
                    state[:, b, c] = (0.0, 0.0, -1e38)
                else:
                    state[:, b, c] = (float(N / exp(top)), float(D / exp(top)), float(top))
    return out, state


def wkv6_brute(lam, k, v, r, H, state_in=None, dps: int = 50):
    """The matrix-valued-state recurrence (oracle/wkv_matrix.py) in 50-digit
    mpmath, written in its attention form: y_t[i] = sigmoid(r_t[i]) times the
    sum over s <= t of exp(-sum_{s<tau<=t} lam_tau[i]) k_s[i] (v_s . k_t), plus
    the initial state's row i applied to k_t and decayed by every step so far.
    No state matrix is formed. Returns y (B, T, C) rounded to float64."""
    lam, k, v, r = (np.asarray(x, dtype=np.float64) for x in (lam, k, v, r))
    B, T, C = k.shape
    D = C // H
    y = np.empty((B, T, C))
    with mpmath.workdps(dps):
        mpf, exp = mpmath.mpf, mpmath.exp
        for b in range(B):
            for h in range(H):
                cs = range(h * D, (h + 1) * D)
                K = [[mpf(k[b, t, c]) for c in cs] for t in range(T)]
                Vv = [[mpf(v[b, t, c]) for c in cs] for t in range(T)]
                Lm = [[mpf(lam[b, t, c]) for c in cs] for t in range(T)]
                for t in range(T):
                    dots = [sum((Vv[s][j] * K[t][j] for j in range(D)), mpf(0)) for s in range(t + 1)]
                    for i in range(D):
                        acc = mpf(0)
                        if state_in is not None:
                            row = sum((mpf(state_in[b, h, i, j]) * K[t][j] for j in range(D)), mpf(0))
                            acc += row * exp(-sum((Lm[tau][i] for tau in range(t + 1)), mpf(0)))
                        for s in range(t + 1):
                            decay = exp(-sum((Lm[tau][i] for tau in range(s + 1, t + 1)), mpf(0)))
                            acc += decay * K[s][i] * dots[s]
                        gate = 1 / (1 + exp(-mpf(r[b, t, h * D + i])))
                        y[b, t, h * D + i] = float(gate * acc)
    return y

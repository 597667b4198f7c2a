"""Float64 CPU oracle for the token shift that feeds the WKV operator's inputs.

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module. It shares no code with the HIP library
and imports nothing from it.

What is computed
----------------
Source: the page "RWKV-v6 Architecture: Attention-Free Linear Transformers",
section "The Core Components of the RWKV-v6 Time-Mixing Block", item 1
"Data-Dependent Token Shift (DD-LERP)" (its four displayed equations); the
page "RWKV: Merging Transformer Training with RNN Speed" (Time-Mixing block)
calls the same blend of each token with the one before it token-shift.

Every projection p (receptance, decay, key, value, ...) gets its own input:
the current token vector moved towards the previous one by a learned
per-channel fraction mu_p,

    x'_p,t = x_t + (x_{t-1} - x_t) * mu_p          (elementwise over channels)

Conventions fixed here (the pages leave them open; every one is listed in the
design notes):

* Shapes: x is (B, T, C), one sequence per batch row; mu is (P, C), one
  mixing vector per projection; the result is (P, B, T, C), the P mixes one
  after the other, each laid out like x.
* x_{t-1} at the first position of a call is the last token of the previous
  call (x_prev, (B, C)); with none, it is the zero vector, as the page's
  listing starts its stream with x_prev = zeros.
* A call also returns the last token of x (the next call's x_prev), so
  prefill and decode chain like the WKV state does.
"""

from __future__ import annotations

import numpy as np


def token_shift(x, mu, x_prev=None):
    """The P mixes of x with its one-token-shifted copy (module docstring).

    x: (B, T, C); mu: (P, C); x_prev: (B, C) or None (zeros). Returns
    (mixes (P, B, T, C), last (B, C)) in float64, last = x[:, T-1] (x_prev
    when T = 0)."""
    x = np.asarray(x, dtype=np.float64)
    mu = np.asarray(mu, dtype=np.float64)
    if x.ndim != 3:
        raise ValueError(f"x must be (B, T, C), got {x.shape}")
    B, T, C = x.shape
    if mu.ndim != 2 or mu.shape[1] != C:
        raise ValueError(f"mu must be (P, {C}), got {mu.shape}")
    prev = np.zeros((B, C)) if x_prev is None else np.asarray(x_prev, dtype=np.float64)
    if prev.shape != (B, C):
        raise ValueError(f"x_prev must be ({B}, {C}), got {prev.shape}")
    # the token before each position: x_prev, then x itself one step behind
    before = np.concatenate([prev[:, None, :], x[:, :-1, :]], axis=1) if T > 0 else x
    mixes = x[None] + (before - x)[None] * mu[:, None, None, :]
    last = x[:, T - 1].copy() if T > 0 else prev.copy()
    return mixes, last

"""Seeded synthetic inputs for the WKV workloads.

This module only draws random numbers and lays them out; it holds none of the
operator's arithmetic. Both the HIP path (through the tests and the benchmark)
and the float64 oracle consume what it produces, so it imports neither.

The pages give no dataset for the operator itself; their model is a 130M
MicroRWKV with 8 layers, embedding width 768 and a 1024-token block (pages
"Linear attention without writing a CUDA kernel", table under
"Configuration", and "MicroRWKV", table under "Configuration"). The workloads
below use those shapes with random activations standing in for that model's
keys and values. Every tensor is drawn from numpy's PCG64 with a seed made of
(workload id, layer, tensor id, batch row), so any batch row of any tensor can
be regenerated alone and the oracle can check a sample of a large run.

Distribution conventions: N(mean, std) uses the standard deviation; a
"log-uniform in [a, b]" decay is exp(U(ln a, ln b)); "1% of entries set to
+-60" is an independent Bernoulli(0.01) mask per entry with a fair sign,
applied before the cast to bf16; bf16 values are rounded to nearest-even from
the float32 draw.
"""

from __future__ import annotations

import concurrent.futures
import dataclasses
import os
from typing import Optional, Sequence, Tuple

import numpy as np

# tensor ids inside a seed
_K, _V, _W, _U, _SPIKE_MASK, _SPIKE_SIGN, _DEC_K, _DEC_V, _GOUT, _R = 1, 2, 3, 4, 5, 6, 7, 8, 9, 10
_WT, _DEC_WT = 11, 12
_SX, _SMU, _SXP = 13, 14, 15


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int                      # workload id (used in every seed)
    name: str
    B: int
    T: int
    C: int
    layers: int = 1
    io: str = "f32"               # "f32" or "bf16" for k, v, out; w, u, state are fp32
    k_kind: str = "normal"        # "normal" (std = k_scale) or "uniform" (+-k_scale)
    k_scale: float = 1.0
    v_std: float = 1.0
    w_lo: float = 0.01
    w_hi: float = 5.0
    u_std: float = 0.5
    spike_p: float = 0.0          # probability that a key is replaced by +-spike_val
    spike_val: float = 60.0
    decode_steps: int = 0         # > 0: a prefill of T tokens, then this many decode steps

    def scaled(self, **kw) -> "Workload":
        """Same distributions and seeds, other sizes (for small parity cases)."""
        return dataclasses.replace(self, **kw)

    @property
    def channel_tokens(self) -> int:
        return self.B * self.T * self.C * self.layers


WORKLOADS = {
    0: Workload(0, "wkv_fwd_B1_T64_C768_f32", B=1, T=64, C=768),
    1: Workload(1, "microrwkv_8x_wkv_fwd_B8_T1024_C768_f32", B=8, T=1024, C=768, layers=8),
    2: Workload(2, "wkv_decode_B256_C768_f32_1024steps_after_T512", B=256, T=512, C=768,
                decode_steps=1024),
    3: Workload(3, "wkv_fwd_long_B4_T16384_C2048_f32", B=4, T=16384, C=2048,
                k_scale=2.0, w_lo=1e-3, w_hi=8.0, u_std=1.0),
    4: Workload(4, "wkv_fwd_stress_B64_T4096_C4096_bf16", B=64, T=4096, C=4096, io="bf16",
                k_kind="uniform", k_scale=20.0, w_lo=1e-3, w_hi=8.0, u_std=1.0,
                spike_p=0.01, spike_val=60.0),
}


def _rng(wl: Workload, layer: int, tensor: int, row: int = 0) -> np.random.Generator:
    return np.random.default_rng([wl.wid, layer, tensor, row])


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 value (ties to even), returned as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    r = np.right_shift(bits, 16)
    np.bitwise_and(r, np.uint32(1), out=r)
    r += np.uint32(0x7FFF)
    r += bits
    np.bitwise_and(r, np.uint32(0xFFFF0000), out=r)
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Exact bf16 values stored in float32 -> their 16-bit patterns (uint16)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    if np.any(bits & np.uint32(0xFFFF)):
        raise ValueError("values are not exactly representable in bf16")
    return np.right_shift(bits, 16).astype(np.uint16)


def _workers(n: int) -> int:
    try:
        cpus = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cpus = os.cpu_count() or 1
    return max(1, min(16, cpus, n))


def _map_rows(fn, rows):
    rows = list(rows)
    if len(rows) <= 1:
        return [fn(r) for r in rows]
    with concurrent.futures.ThreadPoolExecutor(_workers(len(rows))) as ex:
        return list(ex.map(fn, rows))


def params(wl: Workload, layer: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """Per-channel decay w (log-uniform in [w_lo, w_hi]) and bonus u (normal),
    float32, shape (C,)."""
    lo, hi = np.log(wl.w_lo), np.log(wl.w_hi)
    w = np.exp(_rng(wl, layer, _W).uniform(lo, hi, wl.C)).astype(np.float32)
    u = _rng(wl, layer, _U).normal(0.0, wl.u_std, wl.C).astype(np.float32)
    return w, u


def _keys_row(wl: Workload, layer: int, row: int, T: int, tensor: int) -> np.ndarray:
    g = _rng(wl, layer, tensor, row)
    n = T * wl.C
    if wl.k_kind == "normal":
        k = g.standard_normal(n, dtype=np.float32) * np.float32(wl.k_scale)
    elif wl.k_kind == "uniform":
        k = (g.random(n, dtype=np.float32) * np.float32(2 * wl.k_scale)
             - np.float32(wl.k_scale))
    else:
        raise ValueError(wl.k_kind)
    if wl.spike_p > 0 and tensor == _K:
        mask = _rng(wl, layer, _SPIKE_MASK, row).random(n, dtype=np.float32) < wl.spike_p
        sign = _rng(wl, layer, _SPIKE_SIGN, row).integers(0, 2, n, dtype=np.int8)
        k[mask] = np.where(sign[mask] == 1, np.float32(wl.spike_val), np.float32(-wl.spike_val))
    return k.reshape(T, wl.C)


def _values_row(wl: Workload, layer: int, row: int, T: int, tensor: int) -> np.ndarray:
    g = _rng(wl, layer, tensor, row)
    return (g.standard_normal(T * wl.C, dtype=np.float32) * np.float32(wl.v_std)).reshape(T, wl.C)


def kv(wl: Workload, layer: int = 0, rows: Optional[Sequence[int]] = None,
       T: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Prefill keys and values, float32 (B_rows, T, C). For bf16 workloads the
    values are already rounded to bf16 (exactly representable). Rows are drawn
    on a thread pool; each row's stream is independent of the others."""
    rows = list(range(wl.B) if rows is None else rows)
    T = wl.T if T is None else T
    k = np.empty((len(rows), T, wl.C), np.float32)
    v = np.empty((len(rows), T, wl.C), np.float32)

    def one(i):
        kk = _keys_row(wl, layer, rows[i], T, _K)
        vv = _values_row(wl, layer, rows[i], T, _V)
        if wl.io == "bf16":
            kk, vv = round_to_bf16(kk), round_to_bf16(vv)
        k[i] = kk
        v[i] = vv

    _map_rows(one, range(len(rows)))
    return k, v


def decode_kv(wl: Workload, rows: Optional[Sequence[int]] = None,
              steps: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Fresh keys and values for the decode steps, float32 (steps, B_rows, C).
    Keys use the workload's key distribution without spikes."""
    rows = list(range(wl.B) if rows is None else rows)
    steps = wl.decode_steps if steps is None else steps
    k = np.empty((steps, len(rows), wl.C), np.float32)
    v = np.empty((steps, len(rows), wl.C), np.float32)

    def one(i):
        kk = _keys_row(wl, 0, rows[i], steps, _DEC_K)
        vv = _values_row(wl, 0, rows[i], steps, _DEC_V)
        if wl.io == "bf16":
            kk, vv = round_to_bf16(kk), round_to_bf16(vv)
        k[:, i] = kk
        v[:, i] = vv

    _map_rows(one, range(len(rows)))
    return k, v


def grad_out(wl: Workload, layer: int = 0, rows: Optional[Sequence[int]] = None,
             T: Optional[int] = None) -> np.ndarray:
    """Upstream gradient of the prefill output for the backward pass: N(0, 1)
    float32 (B_rows, T, C), one independent stream per batch row."""
    rows = list(range(wl.B) if rows is None else rows)
    T = wl.T if T is None else T
    g = np.empty((len(rows), T, wl.C), np.float32)

    def one(i):
        g[i] = _values_row(wl, layer, rows[i], T, _GOUT)

    _map_rows(one, range(len(rows)))
    return g


def receptance(wl: Workload, layer: int = 0, rows: Optional[Sequence[int]] = None,
               T: Optional[int] = None) -> np.ndarray:
    """Receptance for the gated output: N(0, 1) float32 (B_rows, T, C), rounded
    to bf16 for bf16 workloads, one independent stream per batch row."""
    rows = list(range(wl.B) if rows is None else rows)
    T = wl.T if T is None else T
    r = np.empty((len(rows), T, wl.C), np.float32)

    def one(i):
        rr = _values_row(wl, layer, rows[i], T, _R)
        r[i] = round_to_bf16(rr) if wl.io == "bf16" else rr

    _map_rows(one, range(len(rows)))
    return r


# Per-token decay. The page "RWKV-v6 Architecture: Attention-Free Linear
# Transformers" (section "The Core Components of the RWKV-v6 Time-Mixing
# Block", dynamic data-dependent decay) computes the decay of each token as
# exp(-exp(.)) of a projection of that token; the rate (the inner exp) is then
# a per-channel base times the exponential of a token-dependent term. Here the
# base is the workload's per-channel w and the token term is N(0, 0.5): a
# log-normal modulation, so rates stay positive and spread about 1.6x either
# way around each channel's base.
DD_LOG_STD = 0.5


def decay_rates(wl: Workload, layer: int = 0, rows: Optional[Sequence[int]] = None,
                T: Optional[int] = None) -> np.ndarray:
    """Per-token decay rates (B_rows, T, C) float32: params()' w per channel
    times exp(N(0, DD_LOG_STD)) per entry, rounded to bf16 for bf16 workloads;
    one independent stream per batch row."""
    rows = list(range(wl.B) if rows is None else rows)
    T = wl.T if T is None else T
    wc, _ = params(wl, layer)
    out = np.empty((len(rows), T, wl.C), np.float32)

    def one(i):
        g = _rng(wl, layer, _WT, rows[i])
        z = g.standard_normal(T * wl.C, dtype=np.float32).reshape(T, wl.C)
        r = wc[None, :] * np.exp(np.float32(DD_LOG_STD) * z)
        out[i] = round_to_bf16(r) if wl.io == "bf16" else r

    _map_rows(one, range(len(rows)))
    return out


def decode_decay_rates(wl: Workload, rows: Optional[Sequence[int]] = None,
                       steps: Optional[int] = None) -> np.ndarray:
    """Per-step decay rates for the decode steps (steps, B_rows, C), drawn
    like decay_rates."""
    rows = list(range(wl.B) if rows is None else rows)
    steps = wl.decode_steps if steps is None else steps
    wc, _ = params(wl, 0)
    out = np.empty((steps, len(rows), wl.C), np.float32)

    def one(i):
        g = _rng(wl, 0, _DEC_WT, rows[i])
        z = g.standard_normal(steps * wl.C, dtype=np.float32).reshape(steps, wl.C)
        r = wc[None, :] * np.exp(np.float32(DD_LOG_STD) * z)
        out[:, i] = round_to_bf16(r) if wl.io == "bf16" else r

    _map_rows(one, range(len(rows)))
    return out


# Token shift (the step in front of the projections; page "RWKV-v6
# Architecture: Attention-Free Linear Transformers", section "The Core
# Components of the RWKV-v6 Time-Mixing Block", item 1): the block's input
# vectors stand in as N(0, 1) activations of the workload's width, the
# learned mixing fractions as U(0, 1) per projection and channel.
SHIFT_PROJECTIONS = 4  # receptance, decay, key, value


def shift_inputs(wl: Workload, layer: int = 0, P: int = SHIFT_PROJECTIONS,
                 rows: Optional[Sequence[int]] = None, T: Optional[int] = None):
    """(x (B_rows, T, C), mu (P, C), x_prev (B_rows, C)) float32; x and x_prev
    rounded to bf16 for bf16 workloads; one independent stream per batch
    row."""
    rows = list(range(wl.B) if rows is None else rows)
    T = wl.T if T is None else T
    x = np.empty((len(rows), T, wl.C), np.float32)
    xp = np.empty((len(rows), wl.C), np.float32)

    def one(i):
        xx = _values_row(wl, layer, rows[i], T, _SX)
        pp = _values_row(wl, layer, rows[i], 1, _SXP)[0]
        x[i] = round_to_bf16(xx) if wl.io == "bf16" else xx
        xp[i] = round_to_bf16(pp) if wl.io == "bf16" else pp

    _map_rows(one, range(len(rows)))
    mu = _rng(wl, layer, _SMU).random((P, wl.C), dtype=np.float32)
    return x, mu, xp

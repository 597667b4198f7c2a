"""Helpers shared by the GPU tests: moving seeded inputs to the device, running
the HIP path through the C interface, and comparing with the float64 oracle.

Tolerances (applied elementwise with the oracle's normalised error
|got - ref| / (|ref| + s), s = RMS of v over the tensor):
  * fp32 k, v, out: 1e-5;
  * bf16 k, v, out (fp32 state and arithmetic): 2e-2.
States are compared through their scale-free view (num/den and
max_exp + ln den), since (n, d, m) and (n e^x, d e^x, m - x) are the same state.
"""

from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import canonical, normalised_error, wkv_recurrent, wkv_step_ref
import wkv_recurrence_scan_amd as W
from wkv_recurrence_scan_amd import inputs as I

F32_TOL = 1e-5
BF16_TOL = 2e-2


def say(*a):
    """Print (and flush) what the next GPU step is about to run."""
    print(*a, flush=True)
    sys.stdout.flush()


def dev_f32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def dev_bf16(a) -> torch.Tensor:
    bits = I.bf16_bits(np.asarray(a, dtype=np.float32))
    return torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)


def dev_io(a, io: str) -> torch.Tensor:
    return dev_bf16(a) if io == "bf16" else dev_f32(a)


def host64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def rms(v) -> float:
    v = np.asarray(v, dtype=np.float64)
    return float(np.sqrt(np.mean(v * v))) if v.size else 1.0


def assert_grad_close(got, ref, tol, what, scale=0.0):
    """Elementwise |got - ref| / (|ref| + max(rms(ref), scale)) <= tol: a
    relative error that falls back to the gradient's typical size (or that of
    a companion gradient, `scale`) where an element itself is near zero."""
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite gradient"
    err = np.abs(got - ref) / (np.abs(ref) + max(rms(ref), scale, 1e-30))
    worst = float(err.max()) if err.size else 0.0
    assert worst <= tol, f"{what}: max normalised error {worst:.3e} > {tol:.1e}"
    return worst


def tol_for(io: str) -> float:
    return BF16_TOL if io == "bf16" else F32_TOL


def assert_out_close(got, ref, v, tol, what="out"):
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: {np.size(got) - np.isfinite(got).sum()} non-finite values"
    err = normalised_error(got, ref, max(rms(v), 1e-30))
    worst = float(err.max()) if err.size else 0.0
    assert worst <= tol, f"{what}: max normalised error {worst:.3e} > {tol:.1e} at {np.unravel_index(err.argmax(), err.shape)}"
    return worst


def assert_state_close(got, ref, tol, what="state"):
    got = np.asarray(got, dtype=np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite state"
    rg, Lg = canonical(got)
    rr, Lr = canonical(ref)
    er = np.abs(rg - rr) / (np.abs(rr) + 1.0)
    eL = np.abs(Lg - Lr) / np.maximum(1.0, np.abs(Lr))
    assert er.max() <= tol, f"{what}: num/den error {er.max():.3e} > {tol:.1e}"
    assert eL.max() <= tol, f"{what}: log-denominator error {eL.max():.3e} > {tol:.1e}"
    assert np.all(got[1] > 0), f"{what}: den must stay positive after a token"
    return float(max(er.max(), eL.max()))


def make_case(wl: I.Workload, B: int, T: int, C: int, layer: int = 0):
    """Inputs of workload wl's distributions at another size (host float32)."""
    sw = wl.scaled(B=B, T=T, C=C)
    w, u = I.params(sw, layer)
    k, v = I.kv(sw, layer)
    return w, u, k, v


def random_state(B, C, seed):
    g = np.random.default_rng([99, seed])
    return np.stack([g.normal(0, 1, (B, C)), g.uniform(0.5, 3.0, (B, C)),
                     g.normal(0, 3, (B, C))]).astype(np.float32)


def gpu_forward(w, u, k, v, io="f32", state_in=None, path="auto"):
    """Run the HIP prefill; returns (out, state_out) as float64 host arrays."""
    dw, du = dev_f32(w), dev_f32(u)
    dk, dv = dev_io(k, io), dev_io(v, io)
    ds = None if state_in is None else dev_f32(state_in)
    out, st = W.wkv_forward_ex(dw, du, dk, dv, ds, path=path)
    torch.cuda.synchronize()
    return host64(out), host64(st)


__all__ = [
    "F32_TOL", "BF16_TOL", "say", "dev_f32", "dev_bf16", "dev_io", "host64", "rms", "tol_for",
    "assert_out_close", "assert_state_close", "make_case", "random_state", "gpu_forward",
    "wkv_recurrent", "wkv_step_ref", "W", "I",
]

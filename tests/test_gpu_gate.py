"""GPU parity of the receptance-gated output, out = sigmoid(r) * wkv, for
every prefill kernel, the decode step and the backward pass, against the
float64 oracle (wkv_gated, wkv_gated_backward_direct). Tolerances are those
of the ungated tests: the gate multiplies by a factor in (0, 1) computed to
a few ulp."""

import numpy as np
import pytest
import torch

from oracle import sigmoid, wkv_gated, wkv_gated_backward_direct, wkv_step_ref
from wkvtest import (F32_TOL, I, W, assert_out_close, dev_f32, dev_io, host64, make_case, say,
                     tol_for)

pytestmark = pytest.mark.gpu

WL0, WL3 = I.WORKLOADS[0], I.WORKLOADS[3]
PATHS = ["seq", "chunk", "lookback"]


def receptance(B, T, C, seed=0, scale=2.0):
    return (np.random.default_rng([61, seed, B, T, C]).normal(0, scale, (B, T, C))
            .astype(np.float32))


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("B,T,C", [(1, 1, 8), (2, 37, 40), (1, 300, 32), (2, 1152, 33),
                                   (1, 2500, 70), (64, 40, 256)])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_gated_forward(path, B, T, C, io):
    say(f"gated forward path={path} B={B} T={T} C={C} io={io}")
    w, u, k, v = make_case(WL3, B, T, C)
    r = receptance(B, T, C)
    if io == "bf16":
        k, v, r = (I.round_to_bf16(x) for x in (k, v, r))
    out, st = W.wkv_forward_gated(dev_f32(w), dev_f32(u), dev_io(k, io), dev_io(v, io),
                                  dev_io(r, io), path=path)
    torch.cuda.synchronize()
    ref, rst = wkv_gated(w, u, k, v, r)
    e = assert_out_close(host64(out), ref, v, tol_for(io))
    say(f"  max normalised error {e:.2e}")


def test_gated_forward_extreme_receptance():
    """r = +-100 closes and opens the gate completely without NaN or Inf."""
    B, T, C = 2, 64, 32
    say("gated forward extreme r")
    w, u, k, v = make_case(WL0, B, T, C)
    r = np.where(np.arange(C) % 2 == 0, 100.0, -100.0).astype(np.float32) * np.ones((B, T, 1),
                                                                                    np.float32)
    out, _ = W.wkv_forward_gated(dev_f32(w), dev_f32(u), dev_f32(k), dev_f32(v), dev_f32(r))
    torch.cuda.synchronize()
    got = host64(out)
    ref, _ = wkv_gated(w, u, k, v, r)
    assert np.isfinite(got).all()
    assert np.all(got[:, :, 1::2] == 0.0)
    assert_out_close(got, ref, v, F32_TOL)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_gated_step(io):
    B, C, steps = 4, 96, 6
    say(f"gated step io={io}")
    w, u, k, v = make_case(WL0, B, steps, C)
    r = receptance(B, steps, C, 1)
    if io == "bf16":
        k, v, r = (I.round_to_bf16(x) for x in (k, v, r))
    state = torch.zeros((3, B, C), device="cuda")
    state[2] = -1e38
    st = np.zeros((3, B, C))
    st[2] = -1e38
    for t in range(steps):
        got = W.wkv_step_gated(dev_f32(w), dev_f32(u), dev_io(k[:, t], io), dev_io(v[:, t], io),
                               dev_io(r[:, t], io), state)
        torch.cuda.synchronize()
        ro, st = wkv_step_ref(w, u, k[:, t], v[:, t], st)
        assert_out_close(host64(got), sigmoid(r[:, t]) * ro, v, tol_for(io))


@pytest.mark.parametrize("B,T,C", [(2, 37, 40), (1, 300, 32), (256, 96, 4)])
def test_gated_backward(B, T, C):
    """(2, 37, 40) runs the one-thread-per-lane kernel, (1, 300, 32) and
    (256, 96, 4) the segmented one (every batch row, so dL/dw and dL/du
    are summed over 256 rows)."""
    from test_gpu_backward import assert_grad_close, rms

    say(f"gated backward B={B} T={T} C={C}")
    w, u, k, v = make_case(WL3, B, T, C)
    r = receptance(B, T, C, 2)
    g = np.random.default_rng([62, B, T, C]).normal(0, 1, (B, T, C)).astype(np.float32)
    got = W.wkv_backward(dev_f32(w), dev_f32(u), dev_f32(k), dev_f32(v), dev_f32(g), r=dev_f32(r),
                         want_gstate_in=False)
    torch.cuda.synchronize()
    gw, gu, gk, gv, _, gr = (None if x is None else host64(x) for x in got)
    ref = wkv_gated_backward_direct(w, u, k, v, r, g)
    errs = {}
    for name, a, b, comp in (("gw", gw, ref[0], ref[1]), ("gu", gu, ref[1], ref[0]),
                             ("gk", gk, ref[2], ref[3]), ("gv", gv, ref[3], ref[2]),
                             ("gr", gr, ref[5], ref[3])):
        errs[name] = assert_grad_close(a, b, 1e-4, name, rms(comp))
    say("  " + " ".join(f"{n}={e:.1e}" for n, e in errs.items()))

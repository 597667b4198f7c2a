"""GPU parity of the autograd entry point (wkv_recurrence_scan_amd.wkv: the
checkpoint-saving prefill, then the backward from its checkpoints) against
the float64 gradient oracle (oracle/wkv_grad.py), with the backward tests'
tolerance: ungated and gated, with and without an initial state and a loss
on the final state, sizes over several tiles with ragged ends, and a state
updated in place by a decode step between forward and backward."""

import numpy as np
import pytest
import torch

from oracle import wkv_backward_direct, wkv_gated_backward_direct
from test_gpu_backward import GRAD_TOL, assert_grad_close, rms
from wkvtest import I, W, dev_f32, host64, make_case, random_state, say

pytestmark = pytest.mark.gpu

WL0 = I.WORKLOADS[0]


def leaf(a):
    return dev_f32(a).requires_grad_(True)


def run(B, T, C, gated, with_state, seed, step_after=False):
    say(f"autograd B={B} T={T} C={C} gated={gated} state={with_state} step_after={step_after}")
    w, u, k, v = make_case(WL0, B, T, C, layer=seed)
    g = np.random.default_rng([61, seed])
    r = g.normal(0, 1.5, k.shape).astype(np.float32) if gated else None
    s0 = random_state(B, C, seed) if with_state else None
    gout = g.normal(0, 1, k.shape).astype(np.float32)
    gsn = g.normal(0, 1, (2, B, C)).astype(np.float32)

    tw, tu, tk, tv = leaf(w), leaf(u), leaf(k), leaf(v)
    tr = leaf(r) if gated else None
    ts = leaf(s0) if with_state else None
    out, st = W.wkv(tw, tu, tk, tv, r=tr, state_in=ts)
    st_host = host64(st.detach())
    loss = (out * dev_f32(gout)).sum()
    if with_state:
        loss = loss + (st[:2] * dev_f32(gsn)).sum()
    if step_after:
        # a decode step updates the returned state in place before the backward
        W.wkv_step(tw.detach(), tu.detach(), dev_f32(k[:, 0]), dev_f32(v[:, 0]), st.detach())
    loss.backward()
    torch.cuda.synchronize()

    gs_out = np.concatenate([gsn, np.zeros((1, B, C))]) if with_state else None
    st_ref = st_host if with_state else None
    if gated:
        ref = wkv_gated_backward_direct(w, u, k, v, r, gout, s0, gs_out, st_ref)
    else:
        ref = wkv_backward_direct(w, u, k, v, gout, s0, gs_out, st_ref)
    # the backward tests' companions: each gradient is normalised by the RMS
    # of itself or of its companion, whichever is larger
    companion = {"gw": 1, "gu": 0, "gk": 3, "gv": 2, "gstate_in": 3}
    got = {"gw": tw.grad, "gu": tu.grad, "gk": tk.grad, "gv": tv.grad}
    if with_state:
        got["gstate_in"] = ts.grad
    for i, name in enumerate(("gw", "gu", "gk", "gv", "gstate_in")):
        if name not in got:
            continue
        e = assert_grad_close(host64(got[name]), ref[i], GRAD_TOL, name,
                              rms(ref[companion[name]]))
        say(f"  {name} {e:.2e}")
    if gated:
        e = assert_grad_close(host64(tr.grad), ref[5], GRAD_TOL, "gr")
        say(f"  gr {e:.2e}")


@pytest.mark.parametrize("B,T,C", [(2, 100, 64), (3, 300, 40), (1, 1, 8)])
@pytest.mark.parametrize("gated", [False, True])
def test_autograd_matches_oracle(B, T, C, gated):
    run(B, T, C, gated, with_state=False, seed=B * 1000 + T)


@pytest.mark.parametrize("gated", [False, True])
def test_autograd_with_states(gated):
    run(2, 520, 48, gated, with_state=True, seed=7)


def test_autograd_state_updated_in_place_after_forward():
    run(2, 200, 32, False, with_state=True, seed=9, step_after=True)


def test_autograd_rejects_bf16():
    k = torch.zeros((1, 4, 8), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(8, device="cuda")
    with pytest.raises((ValueError, TypeError)):
        W.wkv(w, w, k, k)

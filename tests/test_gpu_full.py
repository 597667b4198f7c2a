"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times (automatic kernel choice, ForwardCall/StepCall launches):
the GPU runs the whole problem, the oracle recomputes a seeded sample of
(batch row, channel) lanes — lanes are independent, so a sampled lane's
oracle result is exact for that lane. Every output is also checked for
NaN/Inf on the device."""

import numpy as np
import pytest
import torch

from wkvtest import (BF16_TOL, F32_TOL, I, W, assert_out_close, assert_state_close, say,
                     wkv_recurrent, wkv_step_ref)

pytestmark = pytest.mark.gpu


def to_dev(a, io):
    if io == "bf16":
        return torch.from_numpy(I.bf16_bits(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def sample_channels(C, n, seed):
    g = np.random.default_rng([123, seed])
    return np.sort(g.choice(C, size=min(n, C), replace=False))


def check_sampled(wl, layer, out_dev, st_dev, rows, chans, tol):
    w, u = I.params(wl, layer)
    k, v = I.kv(wl, layer, rows=rows)
    k, v = k[:, :, chans], v[:, :, chans]
    ref, rst = wkv_recurrent(w[chans], u[chans], k, v)
    r = torch.as_tensor(rows, device=out_dev.device)
    c = torch.as_tensor(chans, device=out_dev.device)
    got = out_dev.index_select(0, r).index_select(2, c).float().cpu().numpy()
    gst = st_dev.index_select(1, r).index_select(2, c).cpu().numpy()
    e = assert_out_close(got, ref, v, tol, what=f"{wl.name} layer {layer}")
    assert_state_close(gst, rst, F32_TOL * (10 if wl.io == "bf16" else 1),
                       what=f"{wl.name} layer {layer} state")
    return e


def run_full(wl, layer):
    w, u = I.params(wl, layer)
    k, v = I.kv(wl, layer)
    dw, du = to_dev(w, "f32"), to_dev(u, "f32")
    dk, dv = to_dev(k, wl.io), to_dev(v, wl.io)
    del k, v
    call = W.ForwardCall(dw, du, dk, dv)
    out, st = call()
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()), "non-finite outputs"
    assert bool(torch.isfinite(st).all()), "non-finite state"
    return out, st


def test_workload0_full():
    wl = I.WORKLOADS[0]
    say(f"full size: {wl.name}")
    out, st = run_full(wl, 0)
    check_sampled(wl, 0, out, st, list(range(wl.B)), np.arange(wl.C), F32_TOL)


def test_workload1_all_layers_sampled():
    wl = I.WORKLOADS[1]
    say(f"full size: {wl.name} ({W.wkv_select_path(wl.B, wl.T, wl.C)} path)")
    for layer in range(wl.layers):
        out, st = run_full(wl, layer)
        check_sampled(wl, layer, out, st, [0, wl.B - 1], sample_channels(wl.C, 96, layer), F32_TOL)
        del out, st


def test_workload2_prefill_then_1024_decode_steps():
    wl = I.WORKLOADS[2]
    say(f"full size: {wl.name}")
    w, u = I.params(wl)
    k, v = I.kv(wl)
    dk_all, dv_all = I.decode_kv(wl)
    dw, du = to_dev(w, "f32"), to_dev(u, "f32")
    pk, pv = to_dev(k, "f32"), to_dev(v, "f32")
    ks, vs = to_dev(dk_all, "f32"), to_dev(dv_all, "f32")
    _, state = W.ForwardCall(dw, du, pk, pv)()
    outs = torch.empty_like(ks)
    calls = [W.StepCall(dw, du, ks[s], vs[s], state, outs[s]) for s in range(wl.decode_steps)]
    for c in calls:
        c()
    torch.cuda.synchronize()
    assert bool(torch.isfinite(outs).all()) and bool(torch.isfinite(state).all())
    rows = [0, 101, 202, 255]
    _, rs = wkv_recurrent(w, u, k[rows], v[rows])
    ro = []
    for s in range(wl.decode_steps):
        o, rs = wkv_step_ref(w, u, dk_all[s, rows], dv_all[s, rows], rs)
        ro.append(o)
    r = torch.as_tensor(rows, device=outs.device)
    got = outs.index_select(1, r).cpu().numpy()
    assert_out_close(got, np.stack(ro), dv_all[:, rows], F32_TOL, what="decode outputs")
    assert_state_close(state.index_select(1, r).cpu().numpy(), rs, F32_TOL,
                       what="decode final state")


def test_workload3_long_context_sampled():
    wl = I.WORKLOADS[3]
    say(f"full size: {wl.name} ({W.wkv_select_path(wl.B, wl.T, wl.C)} path)")
    out, st = run_full(wl, 0)
    check_sampled(wl, 0, out, st, list(range(wl.B)), sample_channels(wl.C, 128, 3), F32_TOL)


def test_workload4_stress_bf16_sampled():
    wl = I.WORKLOADS[4]
    say(f"full size: {wl.name} ({W.wkv_select_path(wl.B, wl.T, wl.C, W.WKV_IO_BF16)} path)")
    out, st = run_full(wl, 0)
    check_sampled(wl, 0, out, st, [0, 21, 42, 63], sample_channels(wl.C, 128, 4), BF16_TOL)

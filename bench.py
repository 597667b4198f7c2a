#!/usr/bin/env python3
"""Benchmark of the WKV operator on one MI355X.

Default run (one JSON line on stdout):
  * prefill: 8 independent layers of wkv_forward at B=8, T=1024, C=768, fp32
    (the MicroRWKV shape: 8 layers, width 768, 1024-token block), inputs
    resident in HBM. One "step" = the 8 forward calls on one stream, captured
    once into a HIP graph and replayed per step; value = G channel-tokens/s
    over the timed replays. The same steps launched eagerly from Python are
    reported beside it (eager_value).
  * roofline: the prefill kernel's launch duration (HIP events around the
    timed graph replays: step time over launches per step; the eager loop's
    event pair around every launch is reported beside it) against its
    algorithmic HBM bytes (read k, v; write out; write the final state; read
    w, u).
  * decode: 1024 consecutive wkv_step calls at B=256, C=768 after a T=512
    prefill; steps/s for eager launches and for one HIP graph of all 1024.
  * gated_forward: wkv_forward_gated (out = sigmoid(r) * wkv) on one layer of
    the prefill shape.
  * per_token_decay: wkv_forward_dd (a decay rate per token and channel) on
    one layer of the prefill shape and on the decode workload's B=256 T=512
    prefill shape.
  * per_token_decay_backward: wkv_backward_dd (the gradients, a rate per
    token) on the same two shapes, and the training pair with and without
    the checkpoints wkv_forward_dd_ckpt saves.
  * matrix_state: wkv_matrix_forward (a 64 x 64 state per head of 64
    channels) on the same two shapes.
  * backward: wkv_backward (the gradients) on one layer of the prefill shape
    and on the decode workload's B=256 T=512 prefill shape, with the
    roofline on its algorithmic bytes (read k, v, dL/dout; write dL/dk,
    dL/dv).
  * checkpointed_training: on the same two shapes, the plain prefill then
    wkv_backward against wkv_forward_ckpt (the prefill that saves the
    backward's checkpoints) then wkv_backward_ckpt (the backward that reads
    them instead of re-running the recurrence).
  * cpu_baseline: the float64 oracle on the host, on the same prefill workload.

--config N measures another workload (0: B=1 T=64 C=768; 2: the decode
workload's T=512 prefill; 3: B=4 T=16384 C=2048; 4: B=64 T=4096 C=4096 bf16)
in the same format, without the decode part.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "WKV prefill G channel-tokens/s + % HBM roofline; decode steps/s at B=256"
PEAK_HBM_GBS = 8000.0
PEAK_MFMA_F32_TFS = 157.3   # dense fp32 matrix-core peak of MI355X


def _log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(B, T, C, io_bytes, state_in=False):
    """Bytes the operator must move: read k, v and write out (B*T*C each),
    write the final state (3 planes of B*C fp32), read w and u (C fp32 each),
    plus reading an initial state when one is given."""
    b = 3 * io_bytes * B * T * C + 12 * B * C + 8 * C
    return b + (12 * B * C if state_in else 0)


def build_layers(wl, n_layers, dev):
    import torch
    from wkv_recurrence_scan_amd import inputs as I

    layers = []
    for layer in range(n_layers):
        w, u = I.params(wl, layer)
        k, v = I.kv(wl, layer)
        if wl.io == "bf16":
            kd = torch.from_numpy(I.bf16_bits(k).view(np.int16)).to(dev).view(torch.bfloat16)
            vd = torch.from_numpy(I.bf16_bits(v).view(np.int16)).to(dev).view(torch.bfloat16)
        else:
            kd = torch.from_numpy(k).to(dev)
            vd = torch.from_numpy(v).to(dev)
        layers.append(dict(
            w=torch.from_numpy(w).to(dev), u=torch.from_numpy(u).to(dev), k=kd, v=vd,
            out=torch.empty_like(kd),
            st=torch.empty((3, wl.B, wl.C), dtype=torch.float32, device=dev),
            host=(w, u, k, v)))
        del k, v
    return layers


def time_prefill(layers, steps, warmup, path):
    """Times `steps` steps (all layers once each) after `warmup` steps, twice:
    launched eagerly from Python with a HIP event pair around every kernel
    (the per-kernel durations give the roofline figure), and replayed from one
    HIP graph holding a whole step. Returns a dict of timings."""
    import torch
    import wkv_recurrence_scan_amd as W

    stream = torch.cuda.current_stream()
    calls = [W.ForwardCall(L["w"], L["u"], L["k"], L["v"], None, L["out"], L["st"], path=path)
             for L in layers]

    def one_step(evs=None):
        # each call launches on the stream current at call time, which under
        # graph capture is the capturing stream
        for i, c in enumerate(calls):
            if evs is not None:
                evs[i][0].record()
            c()
            if evs is not None:
                evs[i][1].record()

    for _ in range(warmup):
        one_step()
    torch.cuda.synchronize()
    evs = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
            for _ in layers] for _ in range(steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for s in range(steps):
        one_step(evs[s])
    t1.record(stream)
    torch.cuda.synchronize()
    eager_ms = t0.elapsed_time(t1) / steps
    kms = [e0.elapsed_time(e1) for row in evs for (e0, e1) in row]

    eager_out = [(c.out.clone(), c.state_out.clone()) for c in calls]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        one_step()
    for c in calls:
        c.out.zero_()
        c.state_out.zero_()
    g.replay()
    torch.cuda.synchronize()
    for c, (o, st) in zip(calls, eager_out):  # the graph must redo exactly the eager work
        if not (torch.equal(c.out, o) and torch.equal(c.state_out, st)):
            raise RuntimeError("graph replay does not reproduce the eager outputs")
    del eager_out
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(stream)
    for _ in range(steps):
        g.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - wall0) * 1e3 / steps
    graph_ms = t0.elapsed_time(t1) / steps
    return {"graph_ms": graph_ms, "eager_ms": eager_ms, "kernel_ms": float(np.mean(kms)),
            "kernel_ms_median": float(np.median(kms)), "wall_ms": wall_ms}


def time_decode(wl, dev, n_steps, use_graph):
    """1024 wkv_step calls after a T-token prefill; returns steps/s (and the
    average per-step event time in us for the eager run)."""
    import torch
    import wkv_recurrence_scan_amd as W
    from wkv_recurrence_scan_amd import inputs as I

    w, u = I.params(wl)
    k, v = I.kv(wl)
    dk, dv = I.decode_kv(wl, steps=n_steps)
    dw, du = torch.from_numpy(w).to(dev), torch.from_numpy(u).to(dev)
    pk, pv = torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev)
    del k, v
    ks = torch.from_numpy(dk).to(dev)
    vs = torch.from_numpy(dv).to(dev)
    del dk, dv
    outs = torch.empty_like(ks)
    _, st0 = W.wkv_forward(dw, du, pk, pv)
    state = torch.empty_like(st0)
    stream = torch.cuda.current_stream()

    calls = [W.StepCall(dw, du, ks[s], vs[s], state, outs[s]) for s in range(n_steps)]

    def run_all():
        for c in calls:
            c()  # current stream at call time (the capturing stream under capture)

    state.copy_(st0)
    run_all()  # warm-up
    torch.cuda.synchronize()
    res = {}
    state.copy_(st0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    run_all()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    res["steps_per_s"] = n_steps / (ms * 1e-3)
    res["us_per_step"] = ms * 1e3 / n_steps
    if use_graph:
        g = torch.cuda.CUDAGraph()
        state.copy_(st0)
        torch.cuda.synchronize()
        eager_outs = outs.clone()
        with torch.cuda.graph(g):
            run_all()
        torch.cuda.synchronize()
        state.copy_(st0)
        outs.zero_()
        torch.cuda.synchronize()
        g.replay()  # warm-up replay, checked against the eager steps
        torch.cuda.synchronize()
        if not torch.equal(outs, eager_outs):
            raise RuntimeError("decode graph replay does not reproduce the eager steps")
        del eager_outs
        times = []
        for _ in range(5):  # median of five timed replays, each from the same state
            state.copy_(st0)
            torch.cuda.synchronize()
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        gms = float(np.median(times))
        res["graph_steps_per_s"] = n_steps / (gms * 1e-3)
        res["graph_us_per_step"] = gms * 1e3 / n_steps
    bytes_step = 36 * wl.B * wl.C + 8 * wl.C
    res["bytes_per_step"] = bytes_step
    return res


def time_backward(wl, dev, reps=10):
    """wkv_backward (fp32) on workload wl's first layer with a seeded upstream
    gradient: microseconds per call (event pair around `reps` back-to-back
    calls after two warm-up calls) and the roofline on its algorithmic bytes
    (read k, v, dL/dout; write dL/dk, dL/dv; w, u in and dL/dw, dL/du out)."""
    import torch
    import wkv_recurrence_scan_amd as W
    from wkv_recurrence_scan_amd import inputs as I

    w, u = I.params(wl)
    k, v = I.kv(wl)
    g = I.grad_out(wl)
    t = lambda a: torch.from_numpy(a).to(dev)
    dw, du, dk, dv, dg = t(w), t(u), t(k), t(v), t(g)
    del k, v, g
    gk, gv = torch.empty_like(dk), torch.empty_like(dk)
    gw, gu = torch.empty_like(dw), torch.empty_like(dw)
    ws = torch.empty(max(W.wkv_backward_workspace_size(wl.B, wl.T, wl.C), 1), dtype=torch.uint8,
                     device=dev)
    call = lambda: W.wkv_backward(dw, du, dk, dv, dg, want_gstate_in=False, workspace=ws,
                                  out=(gk, gv, gw, gu, None))
    for _ in range(2):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    ct = wl.B * wl.T * wl.C
    abytes = 20 * ct + 16 * wl.C
    achieved = abytes / (us * 1e-6) / 1e9
    return {"workload": f"{wl.name}, one layer, backward", "B": wl.B, "T": wl.T, "C": wl.C,
            "io": "f32",
            "value": round(ct / (us * 1e-6) / 1e9, 3), "unit": "G channel-tokens/s",
            "us_per_call": round(us, 2),
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                         "kernel": "wkv_backward_kernel", "algorithmic_bytes_per_launch": abytes},
            "workspace_bytes": int(ws.numel())}


def time_ckpt_pair(wl, dev, reps=10):
    """A training layer's two calls both ways on workload wl's first layer
    (fp32, seeded inputs and upstream gradient): the plain prefill then
    wkv_backward, which re-runs the recurrence for its own checkpoints, against
    wkv_forward_ckpt, which saves them while it runs, then wkv_backward_ckpt,
    which reads them. Microseconds per call from event pairs around `reps`
    back-to-back calls after two warm-up calls; the roofline of each
    checkpoint call on its algorithmic bytes (the plain call's, plus 16 bytes
    per channel per 8 tokens written by the forward and read by the
    backward)."""
    import torch
    import wkv_recurrence_scan_amd as W
    from wkv_recurrence_scan_amd import inputs as I

    w, u = I.params(wl)
    k, v = I.kv(wl)
    g = I.grad_out(wl)
    t = lambda a: torch.from_numpy(a).to(dev)
    dw, du, dk, dv, dg = t(w), t(u), t(k), t(v), t(g)
    del k, v, g
    out, st = torch.empty_like(dk), torch.empty((3, wl.B, wl.C), device=dev)
    ck = torch.empty(W.ckpt_shape(wl.B, wl.T, wl.C), device=dev)
    gk, gv = torch.empty_like(dk), torch.empty_like(dk)
    gw, gu = torch.empty_like(dw), torch.empty_like(dw)
    ws = torch.empty(max(W.wkv_backward_workspace_size(wl.B, wl.T, wl.C), 1), dtype=torch.uint8,
                     device=dev)
    grads = (gk, gv, gw, gu, None)
    calls = {
        "forward": lambda: W.wkv_forward_ex(dw, du, dk, dv, out=out, state_out=st),
        "backward": lambda: W.wkv_backward(dw, du, dk, dv, dg, want_gstate_in=False,
                                           workspace=ws, out=grads),
        "forward_ckpt": lambda: W.wkv_forward_ckpt(dw, du, dk, dv, out=out, state_out=st,
                                                   ckpt=ck),
        "backward_ckpt": lambda: W.wkv_backward(dw, du, dk, dv, dg, want_gstate_in=False,
                                                workspace=ws, out=grads, ckpt=ck),
    }
    stream = torch.cuda.current_stream()
    us = {}
    for name, call in calls.items():
        for _ in range(2):
            call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        us[name] = e0.elapsed_time(e1) * 1e3 / reps
    ct = wl.B * wl.T * wl.C
    ck_bytes = W.wkv_ckpt_bytes(wl.B, wl.T, wl.C)
    fbytes = 12 * ct + 12 * wl.B * wl.C + 8 * wl.C + ck_bytes
    bbytes = 20 * ct + 16 * wl.C + ck_bytes

    def roof(nbytes, t_us):
        a = nbytes / (t_us * 1e-6) / 1e9
        return {"bound": "hbm", "achieved": round(a, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(a / PEAK_HBM_GBS, 4), "algorithmic_bytes_per_launch": nbytes}

    plain = us["forward"] + us["backward"]
    saved = us["forward_ckpt"] + us["backward_ckpt"]
    return {"workload": f"{wl.name}, one layer, forward then backward", "B": wl.B, "T": wl.T,
            "C": wl.C, "io": "f32", "ckpt_bytes": ck_bytes,
            "us_per_call": {k_: round(x, 2) for k_, x in us.items()},
            "value": round(ct / (saved * 1e-6) / 1e9, 3),
            "plain_value": round(ct / (plain * 1e-6) / 1e9, 3),
            "unit": "G channel-tokens/s (forward + backward)",
            "roofline_forward_ckpt": roof(fbytes, us["forward_ckpt"]),
            "roofline_backward_ckpt": roof(bbytes, us["backward_ckpt"])}


def time_dd_backward(wl, dev, reps=10):
    """wkv_backward_dd (fp32) on workload wl's first layer with per-token
    rates and a seeded upstream gradient: microseconds per call (event pair
    around `reps` calls after two warm-up calls) and the roofline on its
    algorithmic bytes (read w, k, v, dL/dout; write dL/dk, dL/dv, dL/dw; u in
    and dL/du out)."""
    import torch
    import wkv_recurrence_scan_amd as W
    from wkv_recurrence_scan_amd import inputs as I

    _, u = I.params(wl)
    k, v = I.kv(wl)
    g = I.grad_out(wl)
    rates = I.decay_rates(wl)
    t = lambda a: torch.from_numpy(a).to(dev)
    du, dk, dv, dg, dr = t(u), t(k), t(v), t(g), t(rates)
    del k, v, g, rates
    grads = (torch.empty_like(dk), torch.empty_like(dk), torch.empty_like(dk),
             torch.empty_like(du), None)
    ws = torch.empty(max(W.wkv_backward_dd_workspace_size(wl.B, wl.T, wl.C), 1),
                     dtype=torch.uint8, device=dev)
    call = lambda: W.wkv_backward_dd(dr, du, dk, dv, dg, want_gstate_in=False, workspace=ws,
                                     out=grads)
    for _ in range(2):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    # the training pair both ways: the plain prefill then this backward,
    # against the prefill that saves checkpoints then the backward from them
    out, st = torch.empty_like(dk), torch.empty((3, wl.B, wl.C), device=dev)
    ck = torch.empty(W.ckpt_shape(wl.B, wl.T, wl.C), device=dev)
    pair = {
        "forward": lambda: W.wkv_forward_dd(dr, du, dk, dv, out=out, state_out=st),
        "forward_ckpt": lambda: W.wkv_forward_dd_ckpt(dr, du, dk, dv, out=out, state_out=st,
                                                      ckpt=ck),
        "backward_ckpt": lambda: W.wkv_backward_dd(dr, du, dk, dv, dg, want_gstate_in=False,
                                                   workspace=ws, out=grads, ckpt=ck),
    }
    pus = {"backward": us}
    for name, fn in pair.items():
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        pus[name] = e0.elapsed_time(e1) * 1e3 / reps
    ct = wl.B * wl.T * wl.C
    abytes = 28 * ct + 8 * wl.C
    achieved = abytes / (us * 1e-6) / 1e9
    return {"workload": f"{wl.name}, one layer, per-token decay backward", "B": wl.B, "T": wl.T,
            "C": wl.C, "io": "f32",
            "value": round(ct / (us * 1e-6) / 1e9, 3), "unit": "G channel-tokens/s",
            "us_per_call": round(us, 2),
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                         "algorithmic_bytes_per_launch": abytes},
            "workspace_bytes": int(ws.numel()),
            "with_checkpoints": {
                "us_per_call": {k_: round(x, 2) for k_, x in pus.items()},
                "pair_value": round(ct / ((pus["forward_ckpt"] + pus["backward_ckpt"]) * 1e-6)
                                    / 1e9, 3),
                "plain_pair_value": round(ct / ((pus["forward"] + pus["backward"]) * 1e-6) / 1e9,
                                          3),
                "unit": "G channel-tokens/s (forward + backward)"}}


def time_gated(wl, dev, path, reps=50):
    """wkv_forward_gated (out = sigmoid(r) * wkv) on workload wl's first
    layer: microseconds per call from an event pair around `reps`
    back-to-back calls, and the roofline on its algorithmic bytes (read k,
    v, r; write out and the final state; read w, u)."""
    import torch
    import wkv_recurrence_scan_amd as W
    from wkv_recurrence_scan_amd import inputs as I

    w, u = I.params(wl)
    k, v = I.kv(wl)
    r = I.receptance(wl)
    t = lambda a: torch.from_numpy(a).to(dev)
    dw, du, dk, dv, dr = t(w), t(u), t(k), t(v), t(r)
    del k, v, r
    out = torch.empty_like(dk)
    st = torch.empty((3, wl.B, wl.C), dtype=torch.float32, device=dev)
    call = lambda: W.wkv_forward_gated(dw, du, dk, dv, dr, out=out, state_out=st, path=path)
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    ct = wl.B * wl.T * wl.C
    abytes = 16 * ct + 12 * wl.B * wl.C + 8 * wl.C
    achieved = abytes / (us * 1e-6) / 1e9
    return {"workload": f"{wl.name}, one layer, gated output", "path": path,
            "value": round(ct / (us * 1e-6) / 1e9, 3), "unit": "G channel-tokens/s",
            "us_per_call": round(us, 2),
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                         "algorithmic_bytes_per_launch": abytes}}


def time_decay(wl, dev, reps=50):
    """wkv_forward_dd (per-token decay) on workload wl's first layer with the
    seeded per-token rates: microseconds per call from an event pair around
    `reps` back-to-back calls, and the roofline on its algorithmic bytes (read
    w, k, v; write out and the final state; read u)."""
    import torch
    import wkv_recurrence_scan_amd as W
    from wkv_recurrence_scan_amd import inputs as I

    _, u = I.params(wl)
    k, v = I.kv(wl)
    wt = I.decay_rates(wl)
    t = lambda a: torch.from_numpy(a).to(dev)
    dw, du, dk, dv = t(wt), t(u), t(k), t(v)
    del k, v, wt
    out = torch.empty_like(dk)
    st = torch.empty((3, wl.B, wl.C), dtype=torch.float32, device=dev)
    call = lambda: W.wkv_forward_dd(dw, du, dk, dv, out=out, state_out=st)
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    ct = wl.B * wl.T * wl.C
    abytes = 16 * ct + 12 * wl.B * wl.C + 4 * wl.C
    achieved = abytes / (us * 1e-6) / 1e9
    path = W.wkv_select_path(wl.B, wl.T, wl.C, W.WKV_IO_F32)
    return {"workload": f"{wl.name}, one layer, per-token decay", "B": wl.B, "T": wl.T,
            "C": wl.C, "path": "chunk" if path == "lookback" else path,
            "value": round(ct / (us * 1e-6) / 1e9, 3), "unit": "G channel-tokens/s",
            "us_per_call": round(us, 2),
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                         "algorithmic_bytes_per_launch": abytes}}


def time_decode_steps(kind, wl, dev, n_steps=256):
    """Decode steps of the per-token-decay operator (kind "dd": wkv_step_dd)
    or of the matrix-valued state (kind "matrix": wkv_matrix_step) at workload
    wl's batch and width, from the empty state, with the seeded decode
    inputs: the n_steps launches are captured in one HIP graph whose replay
    must reproduce the eager steps; microseconds per step from an event pair
    around one replay, against HBM on the algorithmic bytes per step (dd: read
    w, k, v and the three state planes, write the state and out, read u;
    matrix: read w, k, v, r and the 64 x 64 state per head, write the state
    and out)."""
    import torch
    import wkv_recurrence_scan_amd as W
    from wkv_recurrence_scan_amd import inputs as I

    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    ks, vs = I.decode_kv(wl, steps=n_steps)
    ws = I.decode_decay_rates(wl, steps=n_steps)
    dk, dv, dw = t(ks), t(vs), t(ws)
    del ks, vs, ws
    B, C = wl.B, wl.C
    outs = torch.empty_like(dk)
    if kind == "dd":
        _, u = I.params(wl)
        du = t(u)
        state = torch.empty((3, B, C), dtype=torch.float32, device=dev)

        def reset():
            state[0].zero_()
            state[1].zero_()
            state[2].fill_(-1e38)

        step = lambda s: W.wkv_step_dd(dw[s], du, dk[s], dv[s], state, out=outs[s])
        bytes_step = 40 * B * C + 4 * C
        name = "per-token decay decode step (wkv_step_dd)"
    else:
        H = C // W.MATRIX_HEAD
        rs = I.receptance(wl, layer=1, T=n_steps).transpose(1, 0, 2)
        dr = t(rs)
        del rs
        state = torch.empty((B, H, W.MATRIX_HEAD, W.MATRIX_HEAD), dtype=torch.float32, device=dev)
        reset = state.zero_
        step = lambda s: W.wkv_matrix_step(dw[s], dk[s], dv[s], dr[s], H, state, out=outs[s])
        bytes_step = 20 * B * C + 2 * 4 * B * H * W.MATRIX_HEAD ** 2
        name = f"matrix-valued state decode step (wkv_matrix_step, {H} heads of 64)"

    def run_all():
        for s in range(n_steps):
            step(s)

    reset()
    run_all()
    torch.cuda.synchronize()
    eager = outs.clone()
    g = torch.cuda.CUDAGraph()
    reset()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run_all()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    for _ in range(3):
        reset()
        outs.zero_()
        torch.cuda.synchronize()
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        if not torch.equal(outs, eager):
            raise RuntimeError(f"{kind} decode graph replay does not reproduce the eager steps")
        times.append(e0.elapsed_time(e1) * 1e3 / n_steps)
    us = float(np.median(times))
    achieved = bytes_step / (us * 1e-6) / 1e9
    return {"workload": f"{wl.name}, {name}, from the empty state", "B": B, "C": C,
            "steps": n_steps, "graph_us_per_step": round(us, 3),
            "graph_steps_per_s": round(1e6 / us, 1), "bytes_per_step": bytes_step,
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}}


def time_matrix(wl, dev, reps=20):
    """wkv_matrix_forward (matrix-valued state, heads of 64) on workload wl's
    first layer: k, v, the receptance and the per-token rates of the
    workload, C / 64 heads. Microseconds per call (event pair around `reps`
    back-to-back calls) against two rooflines: HBM on the algorithmic bytes
    (read w, k, v, r; write out and the final state), and the fp32 matrix
    cores on the flops of the chunked form's three contractions per 16-token
    chunk and head of 64 -- the readout S k_t (64 x 64 per token), the state
    update V^T K (64 x 64 per token) and the key-value products v_s . k_t (16
    x 64 per token): 2 (64 + 64 + 16) = 288 flops per channel-token. The
    causal sum inside a chunk runs on the vector units and is not counted."""
    import torch
    import wkv_recurrence_scan_amd as W
    from wkv_recurrence_scan_amd import inputs as I

    H = wl.C // W.MATRIX_HEAD
    k, v = I.kv(wl)
    r = I.receptance(wl)
    lam = I.decay_rates(wl)
    t = lambda a: torch.from_numpy(a).to(dev)
    dl, dk, dv, dr = t(lam), t(k), t(v), t(r)
    del k, v, r, lam
    out = torch.empty_like(dk)
    st = torch.empty((wl.B, H, W.MATRIX_HEAD, W.MATRIX_HEAD), dtype=torch.float32, device=dev)
    nws = W.wkv_matrix_workspace_size(wl.B, wl.T, H)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    call = lambda: W.wkv_matrix_forward(dl, dk, dv, dr, H, out=out, state_out=st, workspace=ws)
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    ct = wl.B * wl.T * wl.C
    abytes = 20 * ct + 4 * wl.B * H * W.MATRIX_HEAD ** 2
    aflops = 2 * (W.MATRIX_HEAD + W.MATRIX_HEAD + 16) * ct
    gbs = abytes / (us * 1e-6) / 1e9
    tfs = aflops / (us * 1e-6) / 1e12
    return {"workload": f"{wl.name}, one layer, matrix-valued state ({H} heads of 64)",
            "B": wl.B, "T": wl.T, "C": wl.C, "heads": H,
            "value": round(ct / (us * 1e-6) / 1e9, 3), "unit": "G channel-tokens/s",
            "us_per_call": round(us, 2), "workspace_bytes": nws,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "algorithmic_bytes_per_launch": abytes},
            "mfma_roofline": {"bound": "mfma", "achieved": round(tfs, 2), "peak": PEAK_MFMA_F32_TFS,
                              "unit": "TFLOP/s", "frac": round(tfs / PEAK_MFMA_F32_TFS, 4),
                              "algorithmic_flops_per_call": aflops}}


def measured_traffic(workload_key, path):
    """HBM bytes per launch from the rocprofv3 counter summaries under
    profiles/ (FETCH_SIZE + WRITE_SIZE, calibrated against a plain copy), or
    None when there is none for this workload and kernel or when the kernel's
    sources have changed since the counters were taken."""
    import glob
    import hashlib

    for f in sorted(glob.glob(os.path.join(ROOT, "profiles", "traffic_*.md"))):
        kv = {}
        for line in open(f):
            if ":" in line and not line.startswith(("|", " ", "#")):
                a, b = line.split(":", 1)
                kv[a.strip()] = b.strip()
        if kv.get("workload_key") != workload_key or kv.get("path") != path:
            continue
        h = hashlib.sha256()
        for src in kv.get("kernel_sources", "").split(","):
            with open(os.path.join(ROOT, src), "rb") as fh:
                h.update(fh.read())
        if h.hexdigest() != kv.get("source_sha256"):
            return None
        return int(kv["traffic_bytes_per_launch"])
    return None


def cpu_baseline(layers, wl, min_s=10.0, budget_s=30.0):
    """The float64 oracle on the host over the benchmarked workload: whole batch
    rows of each layer in turn, in full passes over the workload repeated until
    at least min_s seconds of work are done, or a partial pass cut at about
    budget_s seconds when one pass is longer than that."""
    from oracle import wkv_recurrent

    t0 = time.perf_counter()
    rows_done = 0
    passes = 0
    total_rows = len(layers) * wl.B
    rows_per_call = max(1, min(wl.B, 8192 // wl.C))  # the oracle vectorises over lanes
    cut = False
    while not cut:
        for L in layers:
            w, u, k, v = L["host"]
            for r in range(0, wl.B, rows_per_call):
                r1 = min(wl.B, r + rows_per_call)
                wkv_recurrent(w, u, k[r:r1], v[r:r1])
                rows_done += r1 - r
                if time.perf_counter() - t0 > budget_s:
                    cut = True
                    break
            if cut:
                break
        else:
            passes += 1
        if time.perf_counter() - t0 >= min_s:
            break
    dt = time.perf_counter() - t0
    ct = rows_done * wl.T * wl.C
    what = (f"{passes} full passes over" if rows_done == passes * total_rows
            else f"{rows_done} sequences ({passes} full passes) of")
    return {"value": round(ct / dt / 1e9, 6), "unit": "G channel-tokens/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{what} the {total_rows} (layer, batch-row) sequences of T={wl.T} "
                      f"C={wl.C}; float64 numpy recurrence in one process, {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=1, choices=[0, 1, 2, 3, 4])
    ap.add_argument("--path", default="auto", choices=["auto", "seq", "chunk", "lookback"])
    ap.add_argument("--decode-steps", type=int, default=1024)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the gated, per-token-decay, matrix-state and backward measurements")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one plain device copy of this size (for counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this operator is sharded over (batch, channel) "
              "lanes with no communication, so more GPUs are not part of this benchmark.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import wkv_recurrence_scan_amd as W
    from wkv_recurrence_scan_amd import inputs as I

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    W.load_library()

    wl = I.WORKLOADS[args.config]
    if args.config == 2:
        wl = wl.scaled(decode_steps=0)
    n_layers = wl.layers
    _log(f"generating inputs for {wl.name}")
    layers = build_layers(wl, n_layers, dev)
    io_bytes = 2 if wl.io == "bf16" else 4
    path_used = args.path if args.path != "auto" else W.wkv_select_path(
        wl.B, wl.T, wl.C, W.WKV_IO_BF16 if wl.io == "bf16" else W.WKV_IO_F32)

    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20) // 4
        a = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        _log(f"copy probe: {args.copy_probe_mib} MiB read + {args.copy_probe_mib} MiB written")
        del a, b

    _log(f"timing {args.steps} steps after {args.warmup} warm-up steps, path={path_used}")
    tm = time_prefill(layers, args.steps, args.warmup, args.path)
    ms_step = tm["graph_ms"]
    # Launch duration of the kernel in steady state: HIP events around the
    # timed graph replays, step time over the launches in a step (the gaps
    # between back-to-back launches included). The eager loop's event pair
    # around every single launch also counts the dispatch of each launch and
    # reads a little higher; it is reported beside it.
    kms = ms_step / n_layers
    per_layer_ct = wl.B * wl.T * wl.C
    ct_step = per_layer_ct * n_layers
    value = ct_step / (ms_step * 1e-3) / 1e9
    abytes = algorithmic_bytes(wl.B, wl.T, wl.C, io_bytes)
    achieved = abytes / (kms * 1e-3) / 1e9

    rec = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "G channel-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.io == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "T": wl.T, "C": wl.C, "layers": n_layers,
                   "io": wl.io, "path": path_used, "launch": "hip_graph_per_step",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic(wl.name, path_used),
                     "kernel": f"wkv_{path_used}_kernel", "kernel_us": round(kms * 1e3, 3),
                     "kernel_us_timing": "graph replay events: step time / launches per step",
                     "kernel_us_event_pairs": round(tm["kernel_ms"] * 1e3, 3),
                     "algorithmic_bytes_per_launch": abytes},
        "eager_ms_per_step": round(tm["eager_ms"], 5),
        "eager_value": round(ct_step / (tm["eager_ms"] * 1e-3) / 1e9, 3),
        "wall_ms_per_step": round(tm["wall_ms"], 5),
    }

    if args.config == 1 and not args.no_decode:
        dwl = I.WORKLOADS[2]
        _log(f"decode: {args.decode_steps} steps at B={dwl.B} C={dwl.C} after T={dwl.T}")
        d = time_decode(dwl, dev, args.decode_steps, use_graph=True)
        rec["decode"] = {
            "workload": dwl.name, "B": dwl.B, "C": dwl.C, "prefill_T": dwl.T,
            "steps": args.decode_steps,
            "steps_per_s": round(d["steps_per_s"], 1),
            "us_per_step": round(d["us_per_step"], 3),
            "graph_steps_per_s": round(d.get("graph_steps_per_s", 0.0), 1),
            "graph_us_per_step": round(d.get("graph_us_per_step", 0.0), 3),
            "bytes_per_step": d["bytes_per_step"],
        }

    if args.config == 1 and not args.no_backward:
        _log("gated forward: one layer")
        rec["gated_forward"] = time_gated(wl.scaled(layers=1), dev, path_used)
        rec["backward"] = []
        for bwl in (wl.scaled(layers=1), I.WORKLOADS[2].scaled(decode_steps=0)):
            _log(f"backward: {bwl.name} (one layer)")
            rec["backward"].append(time_backward(bwl, dev))
            torch.cuda.empty_cache()
        rec["checkpointed_training"] = []
        for bwl in (wl.scaled(layers=1), I.WORKLOADS[2].scaled(decode_steps=0)):
            _log(f"checkpointed forward + backward: {bwl.name} (one layer)")
            rec["checkpointed_training"].append(time_ckpt_pair(bwl, dev))
            torch.cuda.empty_cache()

    if args.config == 1 and not args.no_backward:
        rec["per_token_decay"] = []
        for dwl in (wl.scaled(layers=1), I.WORKLOADS[2].scaled(decode_steps=0)):
            _log(f"per-token decay forward: {dwl.name} (one layer)")
            rec["per_token_decay"].append(time_decay(dwl, dev))
            torch.cuda.empty_cache()
        rec["per_token_decay_backward"] = []
        for dwl in (wl.scaled(layers=1), I.WORKLOADS[2].scaled(decode_steps=0)):
            _log(f"per-token decay backward: {dwl.name} (one layer)")
            rec["per_token_decay_backward"].append(time_dd_backward(dwl, dev))
            torch.cuda.empty_cache()

    if args.config == 1 and not args.no_backward:
        rec["matrix_state"] = []
        for mwl in (wl.scaled(layers=1), I.WORKLOADS[2].scaled(decode_steps=0)):
            _log(f"matrix-valued state forward: {mwl.name} (one layer)")
            rec["matrix_state"].append(time_matrix(mwl, dev))
            torch.cuda.empty_cache()

    if args.config == 1 and not args.no_decode and not args.no_backward:
        rec["decode_next"] = []
        for kind in ("dd", "matrix"):
            _log(f"decode steps: {kind} at B={I.WORKLOADS[2].B} C={I.WORKLOADS[2].C}")
            rec["decode_next"].append(time_decode_steps(kind, I.WORKLOADS[2], dev))
            torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        _log("cpu baseline: float64 oracle")
        rec["cpu_baseline"] = cpu_baseline(layers, wl)

    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

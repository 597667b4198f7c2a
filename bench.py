#!/usr/bin/env python3
"""Benchmark of the WKV operator on one MI355X.

Default run (one JSON line on stdout):
  * headline: wkv_forward_bf16 at B=64 T=4096 C=4096 (bf16 k, v, out; fp32
    state and arithmetic), the largest single-GPU workload, inputs resident
    in HBM. One "step" = one prefill call, captured once into a HIP graph and
    replayed per step; value = G channel-tokens/s over the timed replays.
  * roofline: the prefill kernel's launch duration (HIP events on the
    launching stream around the timed graph replays: step time over launches
    per step) against its algorithmic HBM bytes (read k, v; write out; write
    the final state; read w, u), and the HBM traffic from rocprofv3 counter
    summaries under profiles/ when they match the kernel's sources.
  * workloads: the same measurement (value, roofline, traffic) for the other
    prefill workloads: 8 layers of B=8 T=1024 C=768 fp32 (the MicroRWKV
    shape), B=256 T=512 C=768 fp32 (the decode workload's prefill) and
    B=4 T=16384 C=2048 fp32 (long context, through the look-back scan with
    its workspace); the decode workload, 1024 consecutive wkv_step calls at
    B=256 C=768 after a T=512 prefill (steps/s, eager and as one HIP graph);
    and decode time per step after a T=16 prefill against after a T=16384
    prefill (the state is the same size whatever came before).
  * extended: the gated output, the backward pass and the checkpointed
    training pair, per-token decay and its backward, the matrix-valued state,
    the token shift, and the extended operators' decode steps, on the MicroRWKV
    layer shape and the B=256 T=512 shape.
  * cpu_baseline: the float64 oracle on the host's cores, one process per
    core over disjoint lanes, for every workload above (the B=64 T=4096 one on
    4 of its 64 batch rows, scaled to the whole); run before the GPU is
    touched.

--config N puts another workload in the headline (0: B=1 T=64 C=768; 1: the
MicroRWKV layers; 2: B=256 T=512 C=768; 3: B=4 T=16384 C=2048).
--prefill-only measures the prefill workloads alone (for counter runs).
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


def device_layer(wl, layer, dev):
    """w, u, k, v of one layer of workload wl as device tensors (k, v bf16 for
    bf16 workloads), drawn a few batch rows at a time so that host memory
    stays bounded at any size."""
    import torch
    from wkv_recurrence_scan_amd import inputs as I

    w, u = I.params(wl, layer)
    dt = torch.bfloat16 if wl.io == "bf16" else torch.float32
    k = torch.empty((wl.B, wl.T, wl.C), dtype=dt, device=dev)
    v = torch.empty_like(k)
    per = max(1, (1 << 25) // max(1, wl.T * wl.C))  # rows per batch: ~32M elements
    for r0 in range(0, wl.B, per):
        rows = list(range(r0, min(wl.B, r0 + per)))
        kh, vh = I.kv(wl, layer, rows=rows)
        for dst, h in ((k, kh), (v, vh)):
            if wl.io == "bf16":
                dst[r0:r0 + len(rows)] = torch.from_numpy(I.bf16_bits(h).view(np.int16)).to(
                    dev).view(torch.bfloat16)
            else:
                dst[r0:r0 + len(rows)] = torch.from_numpy(h).to(dev)
        del kh, vh
    return dict(w=torch.from_numpy(w).to(dev), u=torch.from_numpy(u).to(dev), k=k, v=v,
                out=torch.empty_like(k),
                st=torch.empty((3, wl.B, wl.C), dtype=torch.float32, device=dev))


def time_prefill(layers, steps, warmup, path="auto"):
    """Times `steps` steps (all layers once each) after `warmup` steps, twice:
    launched eagerly from Python with a HIP event pair around every launch,
    and replayed from one HIP graph holding a whole step (events on the
    launching stream around the timed replays). Every call is a prepared
    ForwardCall that owns the workspace its kernel may need. Returns the
    timings and the calls."""
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
    for c in calls:
        c.check()  # a look-back launch that failed to chain its segments raises
    # non-finite values among the last replay's outputs and final states
    nonfinite = sum(int((~torch.isfinite(c.out)).sum()) + int((~torch.isfinite(c.state_out)).sum())
                    for c in calls)
    return {"graph_ms": graph_ms, "eager_ms": eager_ms, "kernel_ms": float(np.mean(kms)),
            "kernel_ms_median": float(np.median(kms)), "wall_ms": wall_ms,
            "nonfinite": nonfinite}


def prefill_kernel(path, wl):
    """Name of the kernel function a prefill path launches for workload wl
    (the library's launch rules: the bf16 walk stages whole 512-channel row
    pieces through LDS; ungated fp32 chunked scans of two to four 256-token
    tiles whose workgroups of 32 channels each get a CU run two walkers)."""
    import torch

    if path == "seq":
        return "wkv_seq_tile_kernel" if wl.io == "bf16" and wl.C % 512 == 0 else "wkv_seq_kernel"
    if path == "chunk" and wl.io == "f32" and 256 < wl.T <= 1024:
        cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
        if wl.B * -(-wl.C // 32) <= cus:
            return "wkv_chunk_split_kernel"
    return f"wkv_{path}_kernel"


def prefill_record(wl, tm, path):
    """Value and roofline of one timed prefill workload (see time_prefill)."""
    io_bytes = 2 if wl.io == "bf16" else 4
    kms = tm["graph_ms"] / wl.layers
    ct_step = wl.B * wl.T * wl.C * wl.layers
    abytes = algorithmic_bytes(wl.B, wl.T, wl.C, io_bytes)
    achieved = abytes / (kms * 1e-3) / 1e9
    kernel = prefill_kernel(path, wl)
    return {
        "workload": wl.name, "B": wl.B, "T": wl.T, "C": wl.C, "layers": wl.layers, "io": wl.io,
        "path": path, "value": round(ct_step / (tm["graph_ms"] * 1e-3) / 1e9, 3),
        "unit": "G channel-tokens/s", "ms_per_step": round(tm["graph_ms"], 5),
        "eager_value": round(ct_step / (tm["eager_ms"] * 1e-3) / 1e9, 3),
        "nonfinite_outputs": tm["nonfinite"],
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic(wl.name, kernel),
                     "kernel": kernel, "kernel_us": round(kms * 1e3, 3),
                     "kernel_us_timing": "graph replay events: step time / launches per step",
                     "kernel_us_event_pairs": round(tm["kernel_ms"] * 1e3, 3),
                     "algorithmic_bytes_per_launch": abytes},
    }


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


def time_ckpt_pair(wl, dev, reps=10, gated=False):
    """A training layer's two calls both ways on workload wl's first layer
    (fp32, seeded inputs and upstream gradient; with the receptance gate and
    its gradient when `gated`): the plain prefill then
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
    dr = t(I.receptance(wl)) if gated else None
    del k, v, g
    out, st = torch.empty_like(dk), torch.empty((3, wl.B, wl.C), device=dev)
    ck = torch.empty(W.ckpt_shape(wl.B, wl.T, wl.C), device=dev)
    gk, gv = torch.empty_like(dk), torch.empty_like(dk)
    gw, gu = torch.empty_like(dw), torch.empty_like(dw)
    ws = torch.empty(max(W.wkv_backward_workspace_size(wl.B, wl.T, wl.C), 1), dtype=torch.uint8,
                     device=dev)
    grads = (gk, gv, gw, gu, None) + ((torch.empty_like(dk),) if gated else ())
    if gated:
        fwd = lambda: W.wkv_forward_gated(dw, du, dk, dv, dr, out=out, state_out=st)
    else:
        fwd = lambda: W.wkv_forward_ex(dw, du, dk, dv, out=out, state_out=st)
    calls = {
        "forward": fwd,
        "backward": lambda: W.wkv_backward(dw, du, dk, dv, dg, r=dr, want_gstate_in=False,
                                           workspace=ws, out=grads),
        "forward_ckpt": lambda: W.wkv_forward_ckpt(dw, du, dk, dv, dr, out=out, state_out=st,
                                                   ckpt=ck),
        "backward_ckpt": lambda: W.wkv_backward(dw, du, dk, dv, dg, r=dr, want_gstate_in=False,
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
    # the gate adds r to the forward's reads, and r read plus dL/dr written
    # to the backward's
    fbytes = (16 if gated else 12) * ct + 12 * wl.B * wl.C + 8 * wl.C + ck_bytes
    bbytes = (28 if gated else 20) * ct + 16 * wl.C + ck_bytes

    def roof(nbytes, t_us):
        a = nbytes / (t_us * 1e-6) / 1e9
        return {"bound": "hbm", "achieved": round(a, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(a / PEAK_HBM_GBS, 4), "algorithmic_bytes_per_launch": nbytes}

    plain = us["forward"] + us["backward"]
    saved = us["forward_ckpt"] + us["backward_ckpt"]
    gate = ", gated output" if gated else ""
    return {"workload": f"{wl.name}, one layer{gate}, forward then backward", "B": wl.B,
            "T": wl.T, "C": wl.C, "io": "f32", "gated": gated, "ckpt_bytes": ck_bytes,
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
    # the per-token-decay forward's AUTO: the sequential scan wherever B*C
    # lanes give every SIMD a wave (or T < 32), else the chunked scan
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    path = "seq" if wl.T < 32 or -(-wl.B * wl.C // 64) >= 4 * cus else "chunk"
    return {"workload": f"{wl.name}, one layer, per-token decay", "B": wl.B, "T": wl.T,
            "C": wl.C, "path": path,
            "value": round(ct / (us * 1e-6) / 1e9, 3), "unit": "G channel-tokens/s",
            "us_per_call": round(us, 2),
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                         "algorithmic_bytes_per_launch": abytes}}


def time_shift(wl, dev, P=4, reps=50):
    """wkv_token_shift (the P = 4 mixes of each token with the one before it)
    on workload wl's first layer: microseconds per call from an event pair
    around `reps` back-to-back calls, and the roofline on its algorithmic
    bytes (read x once, write P mixes; read mu, x_prev; write x_last)."""
    import torch
    import wkv_recurrence_scan_amd as W
    from wkv_recurrence_scan_amd import inputs as I

    x, mu, xp = I.shift_inputs(wl, P=P)
    dt = torch.bfloat16 if wl.io == "bf16" else torch.float32
    dx = torch.from_numpy(x).to(dev).to(dt)
    dxp = torch.from_numpy(xp).to(dev).to(dt)
    dmu = torch.from_numpy(mu).to(dev)
    del x, xp
    out = torch.empty((P,) + tuple(dx.shape), dtype=dt, device=dev)
    last = torch.empty_like(dxp)
    call = lambda: W.wkv_token_shift(dmu, dx, dxp, out=out, x_last=last)
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
    es = 2 if wl.io == "bf16" else 4
    ct = wl.B * wl.T * wl.C
    abytes = es * (1 + P) * ct + 4 * P * wl.C + 2 * es * wl.B * wl.C
    achieved = abytes / (us * 1e-6) / 1e9
    return {"workload": f"{wl.name}, one layer, token shift", "B": wl.B, "T": wl.T, "C": wl.C,
            "io": wl.io, "projections": P,
            "value": round(ct / (us * 1e-6) / 1e9, 3), "unit": "G channel-tokens/s",
            "us_per_call": round(us, 2),
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                         "kernel": "wkv_shift_kernel", "algorithmic_bytes_per_launch": abytes}}


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


def measured_traffic(workload_key, kernel):
    """HBM bytes per launch of `kernel` on `workload_key` from the rocprofv3
    counter summaries under profiles/ (FETCH_SIZE + WRITE_SIZE, calibrated
    against a plain copy), or None when there is none or when the kernel's
    sources have changed since the counters were taken."""
    import glob
    import hashlib

    for f in sorted(glob.glob(os.path.join(ROOT, "profiles", "traffic_*.md"))):
        kv = {}
        for line in open(f):
            if ":" in line and not line.startswith(("|", " ", "#")):
                a, b = line.split(":", 1)
                kv[a.strip()] = b.strip()
        if kv.get("workload_key") != workload_key or kv.get("kernel") != kernel:
            continue
        h = hashlib.sha256()
        for src in kv.get("kernel_sources", "").split(","):
            with open(os.path.join(ROOT, src), "rb") as fh:
                h.update(fh.read())
        if h.hexdigest() != kv.get("source_sha256"):
            return None
        return int(kv["traffic_bytes_per_launch"])
    return None


def time_decode_after(dev, T, n_steps=1024, seed=5):
    """Decode time per step after a T-token prefill at the decode workload's
    B=256 C=768: the prefill's keys and values are drawn on the device
    (seeded normal), then the decode workload's own 1024 steps run as one HIP
    graph (median of five replays, each from the prefill's state)."""
    import torch
    import wkv_recurrence_scan_amd as W
    from wkv_recurrence_scan_amd import inputs as I

    wl = I.WORKLOADS[2]
    w, u = I.params(wl)
    dw, du = torch.from_numpy(w).to(dev), torch.from_numpy(u).to(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    k = torch.randn((wl.B, T, wl.C), generator=g, device=dev)
    v = torch.randn((wl.B, T, wl.C), generator=g, device=dev)
    _, st0 = W.wkv_forward(dw, du, k, v)
    del k, v
    dk, dv = I.decode_kv(wl, steps=n_steps)
    ks, vs = torch.from_numpy(dk).to(dev), torch.from_numpy(dv).to(dev)
    del dk, dv
    outs = torch.empty_like(ks)
    state = st0.clone()
    calls = [W.StepCall(dw, du, ks[s], vs[s], state, outs[s]) for s in range(n_steps)]
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        for c in calls:
            c()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    for _ in range(6):  # the first replay warms up
        state.copy_(st0)
        torch.cuda.synchronize()
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    us = float(np.median(times[1:])) * 1e3 / n_steps
    return {"prefill_T": T, "graph_us_per_step": round(us, 3),
            "steps_per_s": round(1e6 / us, 1)}


# ------------------------------------------------------------- CPU baseline
#
# The float64 oracle (its stabilised recurrence, numpy, vectorised over the
# lanes it is given) on the host's cores: one process per core, each over a
# disjoint piece of a workload's lanes, its inputs regenerated from the same
# seeds. The processes are forked before the GPU is touched; each draws its
# inputs (not timed), waits at a barrier with the others, then repeats its
# piece until at least CPU_MIN_S seconds have passed; the rate of the whole is
# the sum of the processes' rates.

CPU_MIN_S = 1.0


def _cpu_pieces(cfg, P):
    """Workload cfg's lanes cut into P pieces: for each piece a list of
    (layer, rows, c0, c1) blocks. Workload 4 keeps 4 of its 64 batch rows
    (a sample: every lane costs the same, so the rate is the full one)."""
    from wkv_recurrence_scan_amd import inputs as I

    wl = I.WORKLOADS[2 if cfg == 22 else cfg]
    units = []
    if cfg in (1,):
        units = [(layer, [r], 0, wl.C) for layer in range(wl.layers) for r in range(wl.B)]
    elif cfg in (2, 22):
        units = [(0, [r], 0, wl.C) for r in range(wl.B)]
    else:
        rows = list(range(4)) if cfg == 4 else list(range(wl.B))
        per_row = max(1, -(-P // len(rows)))
        cw = -(-wl.C // per_row)
        units = [(0, [r], c0, min(wl.C, c0 + cw)) for r in rows for c0 in range(0, wl.C, cw)]
    pieces = [[] for _ in range(P)]
    for i, unit in enumerate(units):
        pieces[i * P // len(units)].append(unit)
    return pieces


def _cpu_job(cfg, blocks):
    """Inputs of the blocks (drawn here, not timed) and a function that runs
    the oracle over them once and returns the channel-tokens it covered."""
    from oracle import wkv_recurrent, wkv_step_ref
    from wkv_recurrence_scan_amd import inputs as I

    wl = I.WORKLOADS[2 if cfg == 22 else cfg]
    work = []
    for layer, rows, c0, c1 in blocks:
        w, u = I.params(wl, layer)
        k, v = I.kv(wl, layer, rows=rows)
        k, v = np.ascontiguousarray(k[..., c0:c1]), np.ascontiguousarray(v[..., c0:c1])
        if cfg == 22:
            dk, dv = I.decode_kv(wl, rows=rows, steps=wl.decode_steps)
            _, st = wkv_recurrent(w[c0:c1], u[c0:c1], k, v)
            work.append(("decode", w[c0:c1], u[c0:c1], dk[..., c0:c1], dv[..., c0:c1], st))
        else:
            work.append(("prefill", w[c0:c1], u[c0:c1], k, v, None))

    def run():
        done = 0
        for kind, w, u, a, b, st in work:
            if kind == "prefill":
                wkv_recurrent(w, u, a, b)
                done += a.size
            else:
                for t in range(a.shape[0]):
                    _, st = wkv_step_ref(w, u, a[t], b[t], st)
                done += a.size
        return done

    return run


def _cpu_worker(idx, plan, barrier, queue):
    try:
        for name, cfg, blocks in plan:
            run = _cpu_job(cfg, blocks)
            barrier.wait(timeout=600)
            t0 = time.perf_counter()
            done = passes = 0
            while True:
                done += run()
                passes += 1
                if time.perf_counter() - t0 >= CPU_MIN_S:
                    break
            queue.put((name, idx, done, time.perf_counter() - t0, passes))
    except Exception as e:  # reported by the parent
        queue.put(("error", idx, repr(e), 0.0, 0))


def cpu_baselines(cfgs):
    """{name: cpu_baseline record} for the named workloads (cfg 22 is the
    decode workload's 1024 steps), measured as described above."""
    import multiprocessing as mp
    import platform

    try:
        P = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        P = os.cpu_count() or 1
    P = max(1, min(P, 16))
    ctx = mp.get_context("fork")
    barrier = ctx.Barrier(P)
    queue = ctx.Queue()
    plans = [[] for _ in range(P)]
    for name, cfg in cfgs:
        for i, blocks in enumerate(_cpu_pieces(cfg, P)):
            plans[i].append((name, cfg, blocks))
    procs = [ctx.Process(target=_cpu_worker, args=(i, plans[i], barrier, queue)) for i in range(P)]
    for p in procs:
        p.start()
    results = {}
    for _ in range(P * len(cfgs)):
        name, idx, done, secs, passes = queue.get(timeout=900)
        if name == "error":
            raise RuntimeError(f"cpu baseline worker {idx}: {done}")
        results.setdefault(name, []).append((done, secs, passes))
    for p in procs:
        p.join(timeout=60)
    cpu_model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    out = {}
    for name, cfg in cfgs:
        rs = results[name]
        rate = sum(d / s for d, s, _ in rs)
        passes = min(p for _, _, p in rs)
        sample = {4: "4 of the 64 batch rows (all channels, all 4096 tokens), scaled to the "
                     "whole by the rate",
                  22: "all 196608 lanes of 1024 decode steps after the T=512 prefill (the "
                      "prefill itself not timed)"}.get(cfg, "every lane of the workload")
        unit = "steps/s" if cfg == 22 else "G channel-tokens/s"
        value = rate / (256 * 768) if cfg == 22 else rate / 1e9
        out[name] = {"value": round(value, 6 if cfg != 22 else 2), "unit": unit, "cores": P,
                     "kind": "oracle",
                     "sample": f"{sample}; float64 numpy recurrence, one process per core over "
                               f"disjoint lanes, each repeated >= {CPU_MIN_S:.0f} s "
                               f"(>= {passes} passes)",
                     "cpu": cpu_model}
    return out


def headline_record(records, args):
    """The bench line's headline fields from the first prefill record, with
    the other prefill records as `workloads`."""
    head = records[0]
    rec = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "G channel-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if head["io"] == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": head["workload"], "B": head["B"], "T": head["T"], "C": head["C"],
                   "layers": head["layers"], "io": head["io"], "path": head["path"],
                   "launch": "hip_graph_per_step", "parallelism": "single GPU"},
        "roofline": head["roofline"],
        "eager_value": head["eager_value"],
        "nonfinite_outputs": head["nonfinite_outputs"],
    }
    if head["io"] == "bf16":
        rec["dtype_note"] = "bf16 k, v, out; fp32 state and arithmetic"
    if "cpu_baseline" in head:
        rec["cpu_baseline"] = head["cpu_baseline"]
    rec["workloads"] = records[1:]
    return rec


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50,
                    help="untimed steps before each timed loop (the GPU reaches its steady clocks "
                         "after a few tens of milliseconds of work)")
    ap.add_argument("--config", type=int, default=4, choices=[0, 1, 2, 3, 4])
    ap.add_argument("--decode-steps", type=int, default=1024)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the extended measurements (gate, backward, per-token decay, "
                         "matrix state, token shift)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only the prefill workloads (no decode, extended or CPU baseline)")
    ap.add_argument("--extended-only", action="store_true",
                    help="only the extended measurements (for counter runs of their kernels; the "
                         "line then carries no headline)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one plain device copy of this size (for counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this operator is sharded over (batch, channel) "
              "lanes with no communication, so more GPUs are not part of this benchmark.",
              file=sys.stderr)
        sys.exit(2)
    if args.prefill_only:
        args.no_decode = args.no_backward = args.no_cpu_baseline = True
    if args.extended_only:
        args.no_decode = args.no_cpu_baseline = True

    from wkv_recurrence_scan_amd import inputs as I

    prefill_cfgs = [args.config] + [c for c in (1, 2, 3, 4) if c != args.config]
    names = {c: I.WORKLOADS[c].name for c in (0, 1, 2, 3, 4)}
    names[2] = "wkv_fwd_B256_T512_C768_f32"
    cpu = {}
    if not args.no_cpu_baseline:
        # before anything touches the GPU: the workers are forked
        _log("cpu baseline: float64 oracle on the host cores")
        cfgs = [(names[c], c) for c in prefill_cfgs] + ([] if args.no_decode else
                                                       [(I.WORKLOADS[2].name, 22)])
        cpu = cpu_baselines(cfgs)

    import torch
    import wkv_recurrence_scan_amd as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    W.load_library()

    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20) // 4
        a = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        _log(f"copy probe: {args.copy_probe_mib} MiB read + {args.copy_probe_mib} MiB written")
        del a, b

    records = []
    for c in ([] if args.extended_only else prefill_cfgs):
        wl = I.WORKLOADS[c]
        if c == 2:
            wl = wl.scaled(decode_steps=0, name=names[2])
        path = W.wkv_select_path(wl.B, wl.T, wl.C, W.WKV_IO_BF16 if wl.io == "bf16" else W.WKV_IO_F32)
        _log(f"prefill {wl.name}: generating inputs")
        layers = [device_layer(wl, layer, dev) for layer in range(wl.layers)]
        _log(f"prefill {wl.name}: {args.steps} steps after {args.warmup} warm-up steps, path={path}")
        tm = time_prefill(layers, args.steps, args.warmup)
        rec = prefill_record(wl, tm, path)
        if names[c] in cpu:
            rec["cpu_baseline"] = cpu[names[c]]
        records.append(rec)
        del layers
        torch.cuda.empty_cache()

    if args.extended_only:
        rec = {"metric": METRIC, "note": "extended measurements only (no headline)"}
    else:
        rec = headline_record(records, args)

    if not args.no_decode:
        dwl = I.WORKLOADS[2]
        _log(f"decode: {args.decode_steps} steps at B={dwl.B} C={dwl.C} after T={dwl.T}")
        d = time_decode(dwl, dev, args.decode_steps, use_graph=True)
        bstep = d["bytes_per_step"]
        gus = d.get("graph_us_per_step", 0.0)
        dec = {
            "workload": dwl.name, "B": dwl.B, "C": dwl.C, "prefill_T": dwl.T,
            "steps": args.decode_steps, "value": round(d.get("graph_steps_per_s", 0.0), 1),
            "unit": "steps/s", "launch": "one HIP graph of all steps",
            "graph_us_per_step": round(gus, 3),
            "eager_steps_per_s": round(d["steps_per_s"], 1),
            "eager_us_per_step": round(d["us_per_step"], 3),
            "roofline": {"bound": "hbm", "achieved": round(bstep / (gus * 1e-6) / 1e9, 1),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(bstep / (gus * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                         "kernel": "wkv_step_kernel", "algorithmic_bytes_per_step": bstep,
                         "note": "launch-bound: each step's own HBM time is under 1 us"},
        }
        if dwl.name in cpu:
            dec["cpu_baseline"] = cpu[dwl.name]
        rec["decode"] = dec
        torch.cuda.empty_cache()
        _log("decode after a T=16 and a T=16384 prefill")
        flat = [time_decode_after(dev, T) for T in (16, 16384)]
        torch.cuda.empty_cache()
        rec["decode_vs_prefill_length"] = {
            "B": dwl.B, "C": dwl.C, "steps": args.decode_steps, "runs": flat,
            "ratio_long_to_short": round(flat[1]["graph_us_per_step"]
                                         / flat[0]["graph_us_per_step"], 4)}

    if not args.no_backward:
        wl1 = I.WORKLOADS[1]
        path1 = W.wkv_select_path(wl1.B, wl1.T, wl1.C)
        ext = {}
        _log("gated forward: one layer")
        ext["gated_forward"] = time_gated(wl1.scaled(layers=1), dev, path1)
        shapes = (wl1.scaled(layers=1), I.WORKLOADS[2].scaled(decode_steps=0))
        ext["backward"] = []
        for bwl in shapes:
            _log(f"backward: {bwl.name} (one layer)")
            ext["backward"].append(time_backward(bwl, dev))
            torch.cuda.empty_cache()
        ext["checkpointed_training"] = []
        for bwl in shapes:
            _log(f"checkpointed forward + backward: {bwl.name} (one layer)")
            ext["checkpointed_training"].append(time_ckpt_pair(bwl, dev))
            torch.cuda.empty_cache()
        _log(f"checkpointed forward + backward, gated: {shapes[0].name} (one layer)")
        ext["checkpointed_training"].append(time_ckpt_pair(shapes[0], dev, gated=True))
        torch.cuda.empty_cache()
        ext["per_token_decay"] = []
        for dwl_ in shapes:
            _log(f"per-token decay forward: {dwl_.name} (one layer)")
            ext["per_token_decay"].append(time_decay(dwl_, dev))
            torch.cuda.empty_cache()
        ext["per_token_decay_backward"] = []
        for dwl_ in shapes:
            _log(f"per-token decay backward: {dwl_.name} (one layer)")
            ext["per_token_decay_backward"].append(time_dd_backward(dwl_, dev))
            torch.cuda.empty_cache()
        ext["matrix_state"] = []
        for mwl in shapes:
            _log(f"matrix-valued state forward: {mwl.name} (one layer)")
            ext["matrix_state"].append(time_matrix(mwl, dev))
            torch.cuda.empty_cache()
        ext["token_shift"] = []
        for swl in (wl1.scaled(layers=1), I.WORKLOADS[4].scaled(layers=1)):
            _log(f"token shift: {swl.name} (one layer, 4 projections)")
            ext["token_shift"].append(time_shift(swl, dev))
            torch.cuda.empty_cache()
        if not args.no_decode:
            ext["decode_next"] = []
            for kind in ("dd", "matrix"):
                _log(f"decode steps: {kind} at B={I.WORKLOADS[2].B} C={I.WORKLOADS[2].C}")
                ext["decode_next"].append(time_decode_steps(kind, I.WORKLOADS[2], dev))
                torch.cuda.empty_cache()
        rec["extended"] = ext

    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

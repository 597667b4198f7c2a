"""HIP-graph capture and concurrent host threads for the extended operators.

* The per-token-decay and matrix-valued-state prefill, followed by decode
  steps, captured once in a HIP graph: every replay (outputs cleared and the
  decode state reset in between, with unrelated eager work between replays)
  reproduces the eager results bit for bit. The matrix call uses segments,
  so two kernels and the workspace are inside the graph.
* The library is documented as thread-safe: four host threads, each with its
  own stream and buffers, run the constant-decay, per-token-decay and
  matrix-state prefill side by side; every result equals the one computed
  alone beforehand, bit for bit."""

import threading

import numpy as np
import pytest
import torch

from wkvtest import I, W, dev_f32, say

pytestmark = pytest.mark.gpu


def bits(t):
    return t.contiguous().view(torch.int32)


def test_decay_prefill_and_steps_in_hip_graph():
    say("per-token decay graph capture")
    wl = I.WORKLOADS[1].scaled(B=2, T=300, C=96)
    _, u = I.params(wl)
    k, v = I.kv(wl)
    rates = I.decay_rates(wl)
    dk, dv = I.decode_kv(wl, steps=5)
    drt = I.decode_decay_rates(wl, steps=5)
    du, k, v, rates = dev_f32(u), dev_f32(k), dev_f32(v), dev_f32(rates)
    dk, dv, drt = dev_f32(dk), dev_f32(dv), dev_f32(drt)
    out = torch.empty_like(k)
    st = torch.empty((3, wl.B, wl.C), device="cuda")
    step_out = torch.empty((5, wl.B, wl.C), device="cuda")

    def run():
        W.wkv_forward_dd(rates, du, k, v, out=out, state_out=st)
        for s in range(5):
            W.wkv_step_dd(drt[s], du, dk[s], dv[s], st, out=step_out[s])

    run()
    torch.cuda.synchronize()
    eager = [out.clone(), st.clone(), step_out.clone()]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        out.zero_()
        st.zero_()
        step_out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, ref in zip((out, st, step_out), eager):
            assert torch.equal(bits(got), bits(ref)), f"replay {rep}"
        _ = W.wkv_forward_dd(rates, du, k, v)  # unrelated eager work


def test_matrix_prefill_and_steps_in_hip_graph():
    say("matrix state graph capture")
    B, T, H = 1, 700, 2
    wl = I.WORKLOADS[1].scaled(B=B, T=T, C=H * 64)
    k, v = I.kv(wl, 2)
    r = I.receptance(wl, 2)
    lam = I.decay_rates(wl, 2)
    lam, k, v, r = dev_f32(lam), dev_f32(k), dev_f32(v), dev_f32(r)
    nws = W.wkv_matrix_workspace_size(B, T, H)
    assert nws > 0, "this shape should use segments"
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(k)
    st = torch.empty((B, H, 64, 64), device="cuda")
    step_out = torch.empty((4, B, H * 64), device="cuda")
    steps = [(lam[:, t].contiguous(), k[:, t].contiguous(), v[:, t].contiguous(),
              r[:, t].contiguous()) for t in range(4)]

    def run():
        W.wkv_matrix_forward(lam, k, v, r, H, out=out, state_out=st, workspace=ws)
        for s, (a, b, c, d) in enumerate(steps):
            W.wkv_matrix_step(a, b, c, d, H, st, out=step_out[s])

    run()
    torch.cuda.synchronize()
    eager = [out.clone(), st.clone(), step_out.clone()]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        out.zero_()
        st.zero_()
        step_out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, ref in zip((out, st, step_out), eager):
            assert torch.equal(bits(got), bits(ref)), f"replay {rep}"
        _ = W.wkv_matrix_forward(lam, k, v, r, H)  # unrelated eager work


def test_concurrent_host_threads_match_serial_results():
    say("four host threads, own streams")
    nthreads, reps = 4, 5
    cases = []
    for i in range(nthreads):
        wl = I.WORKLOADS[1].scaled(B=2, T=257 + 64 * i, C=128)
        w, u = I.params(wl, i)
        k, v = I.kv(wl, i)
        rates = I.decay_rates(wl, i)
        r = I.receptance(wl, i)
        cases.append(dict(w=dev_f32(w), u=dev_f32(u), k=dev_f32(k), v=dev_f32(v),
                          rates=dev_f32(rates), r=dev_f32(r)))

    def run(c, stream):
        a = W.wkv_forward_ex(c["w"], c["u"], c["k"], c["v"], path="chunk", stream=stream)
        b = W.wkv_forward_dd(c["rates"], c["u"], c["k"], c["v"], stream=stream)
        m = W.wkv_matrix_forward(c["rates"], c["k"], c["v"], c["r"], 2, stream=stream)
        return [t for pair in (a, b, m) for t in pair]

    serial = []
    for c in cases:
        serial.append([t.clone() for t in run(c, torch.cuda.current_stream())])
    torch.cuda.synchronize()

    results = [None] * nthreads
    errors = []

    def worker(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(reps):
                    got = run(cases[i], s)
                s.synchronize()
            results[i] = [t.clone() for t in got]
        except Exception as e:  # reported by the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(nthreads)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not errors, errors
    assert all(not t.is_alive() for t in threads)
    torch.cuda.synchronize()
    for i in range(nthreads):
        for got, ref in zip(results[i], serial[i]):
            assert torch.equal(bits(got), bits(ref)), f"thread {i}"

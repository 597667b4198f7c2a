"""Parity of the HIP path (through the C interface) with the float64 oracle,
element by element, on seeded inputs small enough for the oracle: ragged
sizes around every tile edge of both prefill kernels, initial states,
in-place states, split/resume, decode, bf16 I/O and extreme keys."""

import numpy as np
import pytest
import torch

from wkvtest import (BF16_TOL, F32_TOL, I, W, assert_out_close, assert_state_close, dev_f32,
                     dev_io, gpu_forward, host64, make_case, random_state, say, tol_for,
                     wkv_recurrent, wkv_step_ref)

pytestmark = pytest.mark.gpu

PATHS = ["seq", "chunk", "lookback"]
WL0 = I.WORKLOADS[0]   # k, v ~ N(0, 1), w in [0.01, 5], u ~ N(0, 0.5)
WL3 = I.WORKLOADS[3]   # k ~ N(0, 2), w in [1e-3, 8] (slow and fast decays), u ~ N(0, 1)
WL4 = I.WORKLOADS[4]   # bf16, k ~ U(-20, 20) with 1% +-60 spikes

# T around the chunked kernel's tiles (64 tokens for T <= 256, 256 up to
# T = 2048, 128 beyond; its workgroup shape changes at T = 256 and T = 2048) and the look-back kernel's
# segments (32 tokens for T <= 512, else 128; anchors every 8 segments), and C
# around both kernels' 32-channel groups (64 for bf16); every kernel runs every
# shape.
SHAPES = [
    (1, 1, 1), (2, 2, 7), (1, 3, 16), (3, 31, 33), (2, 32, 5), (2, 63, 48), (2, 64, 64),
    (2, 65, 17), (1, 255, 16), (1, 256, 32), (1, 257, 80), (2, 511, 24), (1, 1000, 40),
    (1, 2048, 31), (1, 2049, 96), (2, 3000, 100), (1, 4097, 16), (1, 513, 40), (2, 1152, 33),
    (1, 1153, 64),
]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("B,T,C", SHAPES)
@pytest.mark.parametrize("wl", [WL0, WL3], ids=["dist0", "dist3"])
def test_forward_f32(path, B, T, C, wl):
    say(f"forward f32 path={path} B={B} T={T} C={C} wl={wl.wid}")
    w, u, k, v = make_case(wl, B, T, C)
    got, gst = gpu_forward(w, u, k, v, "f32", path=path)
    ref, rst = wkv_recurrent(w, u, k, v)
    assert_out_close(got, ref, v, F32_TOL)
    assert_state_close(gst, rst, F32_TOL)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("B,T,C", [(1, 1, 2), (2, 3, 6), (2, 65, 34), (1, 257, 64),
                                   (3, 700, 32), (1, 2049, 66), (1, 130, 7), (1, 2500, 130)])
def test_forward_bf16(path, B, T, C):
    say(f"forward bf16 path={path} B={B} T={T} C={C}")
    w, u, k, v = make_case(WL4, B, T, C)
    got, gst = gpu_forward(w, u, k, v, "bf16", path=path)
    ref, rst = wkv_recurrent(w, u, k, v)
    assert_out_close(got, ref, v, BF16_TOL)
    assert_state_close(gst, rst, F32_TOL * 10)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_forward_from_initial_state(path, io):
    B, T, C = 2, 300, 48
    say(f"initial state path={path} io={io}")
    w, u, k, v = make_case(WL4 if io == "bf16" else WL3, B, T, C)
    s0 = random_state(B, C, 1)
    got, gst = gpu_forward(w, u, k, v, io, state_in=s0, path=path)
    ref, rst = wkv_recurrent(w, u, k, v, s0.astype(np.float64))
    assert_out_close(got, ref, v, tol_for(io))
    assert_state_close(gst, rst, F32_TOL * (10 if io == "bf16" else 1))


@pytest.mark.parametrize("path", PATHS)
def test_state_in_place(path):
    B, T, C = 2, 200, 32
    say(f"in-place state path={path}")
    w, u, k, v = make_case(WL3, B, T, C)
    s0 = random_state(B, C, 2)
    ds = dev_f32(s0)
    out, st = W.wkv_forward_ex(dev_f32(w), dev_f32(u), dev_f32(k), dev_f32(v), ds, state_out=ds,
                               path=path)
    torch.cuda.synchronize()
    assert st is ds
    ref, rst = wkv_recurrent(w, u, k, v, s0.astype(np.float64))
    assert_out_close(host64(out), ref, v, F32_TOL)
    assert_state_close(host64(ds), rst, F32_TOL)


@pytest.mark.parametrize("path", PATHS)
def test_split_and_resume(path):
    B, T, C = 2, 777, 40
    say(f"split/resume path={path}")
    w, u, k, v = make_case(WL3, B, T, C)
    ref, rst = wkv_recurrent(w, u, k, v)
    for cut in (1, 300, 776):
        o1, s1 = gpu_forward(w, u, k[:, :cut], v[:, :cut], path=path)
        o2, s2 = gpu_forward(w, u, k[:, cut:], v[:, cut:], state_in=s1.astype(np.float32),
                             path=path)
        assert_out_close(np.concatenate([o1, o2], axis=1), ref, v, F32_TOL)
        assert_state_close(s2, rst, F32_TOL)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_step_matches_oracle_and_forward(io):
    B, T, C = 3, 96, 36
    say(f"decode steps io={io}")
    w, u, k, v = make_case(WL4 if io == "bf16" else WL0, B, T, C)
    ref, rst = wkv_recurrent(w, u, k, v)
    dw, du = dev_f32(w), dev_f32(u)
    state = dev_f32(np.stack([np.zeros((B, C)), np.zeros((B, C)), np.full((B, C), -1e38)]))
    outs = []
    for t in range(T):
        outs.append(W.step(dw, du, dev_io(k[:, t], io), dev_io(v[:, t], io), state))
    torch.cuda.synchronize()
    got = np.stack([host64(o) for o in outs], axis=1)
    assert_out_close(got, ref, v, tol_for(io))
    assert_state_close(host64(state), rst, F32_TOL * (10 if io == "bf16" else 1))


def test_decode_after_prefill_scaled():
    """The decode workload at reduced size: a prefill, then many steps."""
    wl = I.WORKLOADS[2]
    B, T, C, steps = 4, 512, 64, 300
    say(f"decode after prefill B={B} T={T} C={C} steps={steps}")
    sw = wl.scaled(B=B, T=T, C=C)
    w, u = I.params(sw)
    k, v = I.kv(sw)
    dk, dv = I.decode_kv(sw, steps=steps)
    dw, du = dev_f32(w), dev_f32(u)
    _, st = W.wkv_forward(dw, du, dev_f32(k), dev_f32(v))
    outs = [W.wkv_step(dw, du, dev_f32(dk[s]), dev_f32(dv[s]), st) for s in range(steps)]
    torch.cuda.synchronize()
    _, rs = wkv_recurrent(w, u, k, v)
    ro = []
    for s in range(steps):
        o, rs = wkv_step_ref(w, u, dk[s], dv[s], rs)
        ro.append(o)
    assert_out_close(np.stack([host64(o) for o in outs]), np.stack(ro), dv, F32_TOL)
    assert_state_close(host64(st), rs, F32_TOL)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_deterministic(path, io):
    B, T, C = 2, 600, 64
    say(f"determinism path={path} io={io}")
    w, u, k, v = make_case(WL4 if io == "bf16" else WL3, B, T, C)
    dk, dv, dw, du = dev_io(k, io), dev_io(v, io), dev_f32(w), dev_f32(u)
    o1, s1 = W.wkv_forward_ex(dw, du, dk, dv, path=path)
    o2, s2 = W.wkv_forward_ex(dw, du, dk, dv, path=path)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16) if io == "bf16" else o1.view(torch.int32),
                       o2.view(torch.int16) if io == "bf16" else o2.view(torch.int32))
    assert torch.equal(s1.view(torch.int32), s2.view(torch.int32))


def ulp32(x: float) -> float:
    """Spacing of float32 numbers at magnitude x."""
    return float(np.spacing(np.float32(x)))


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("kmag", [60.0, 88.0, 1e4])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_extreme_keys(path, kmag, io):
    """No NaN/Inf and oracle agreement with keys far outside N(0, 1). An fp32
    exponent of size |k| is only known to ulp(|k|), which moves a weight by
    that much relative, so the bound is the larger of the workload tolerance
    and 4 ulp(|k|): 1.5e-5 at |k| = 60, 3.1e-5 at 88, 3.9e-3 at 1e4."""
    B, T, C = 2, 300, 32
    say(f"extreme keys path={path} k=+-{kmag} io={io}")
    g = np.random.default_rng([7, int(kmag)])
    w, u, _, v = make_case(WL3, B, T, C)
    k = g.choice(np.array([-kmag, kmag, 0.0, 1.0, -3.0], dtype=np.float32), size=(B, T, C))
    if io == "bf16":
        v = I.round_to_bf16(v)
        k = I.round_to_bf16(k)
    got, gst = gpu_forward(w, u, k, v, io, path=path)
    ref, rst = wkv_recurrent(w, u, k, v)
    tol = max(tol_for(io), 4 * ulp32(kmag))
    e = assert_out_close(got, ref, v, tol)
    say(f"  max normalised output error {e:.3e} (bound {tol:.1e})")
    assert np.isfinite(gst).all()
    assert_state_close(gst, rst, max(F32_TOL, 4 * ulp32(kmag)))


def test_auto_path_choice():
    """Large B*C goes to the sequential scan; small B*C to the chunked scan up
    to T = 2048 and to the look-back scan beyond (the chunked scan when no
    workspace is given)."""
    assert W.wkv_select_path(256, 512, 768) == "seq"
    assert W.wkv_select_path(64, 4096, 4096, W.WKV_IO_BF16) == "seq"
    assert W.wkv_select_path(8, 1024, 768) == "chunk"
    assert W.wkv_select_path(4, 16384, 2048) == "lookback"
    assert W.wkv_select_path(1, 64, 768) == "chunk"
    assert W.wkv_select_path(4, 8, 64) == "seq"


def test_lookback_workspace_counters_and_error_word():
    """The look-back kernel's workspace after n launches: every channel
    group's ticket counter advanced by exactly S (segments per group) per
    launch, which is what gives each launch its own epoch, and the error word
    (set only if a bounded wait timed out) still zero. T = 3000 uses
    256-token segments, so S = 12."""
    wl = WL3.scaled(B=2, T=3000, C=96)
    w, u = I.params(wl)
    k, v = I.kv(wl)
    ws = W.new_workspace(W.wkv_workspace_size(2, 3000, 96, W.WKV_IO_F32, "lookback"), "cuda")
    say("look-back workspace counters")
    ref, _ = wkv_recurrent(w, u, k, v)
    groups, S = 2 * ((96 + 31) // 32), (3000 + 255) // 256
    for n in range(3):
        out, _ = W.wkv_forward_ws(dev_f32(w), dev_f32(u), dev_f32(k), dev_f32(v), path="lookback",
                                  workspace=ws)
        torch.cuda.synchronize()
        assert_out_close(host64(out), ref, v, F32_TOL)
        words = ws[:16 + 16 * groups].view(torch.int64).cpu().numpy()
        assert int(words[0]) & 0xffffffff == 0, "a bounded wait timed out"
        tickets = words[2:].reshape(groups, 2)[:, 0]
        assert np.all(tickets == (n + 1) * S), tickets


def test_decode_in_hip_graph_replays_match_eager():
    """Decode steps captured once in a HIP graph give bit-identical results to
    the same steps launched eagerly, on every replay (eager work in between)."""
    wl = I.WORKLOADS[2].scaled(B=8, T=64, C=128)
    steps = 16
    say("decode graph capture")
    w, u = I.params(wl)
    k, v = I.kv(wl)
    dk, dv = I.decode_kv(wl, steps=steps)
    dw, du = dev_f32(w), dev_f32(u)
    ks, vs = dev_f32(dk), dev_f32(dv)
    _, st0 = W.wkv_forward(dw, du, dev_f32(k), dev_f32(v))
    state = st0.clone()
    eager = torch.empty_like(ks)
    for s in range(steps):
        W.wkv_step(dw, du, ks[s], vs[s], state, eager[s])
    eager_state = state.clone()
    outs = torch.empty_like(ks)
    g = torch.cuda.CUDAGraph()
    state.copy_(st0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for s in range(steps):
            W.wkv_step(dw, du, ks[s], vs[s], state, outs[s])
    for rep in range(3):
        state.copy_(st0)
        outs.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(outs.view(torch.int32), eager.view(torch.int32)), f"replay {rep}"
        assert torch.equal(state.view(torch.int32), eager_state.view(torch.int32)), f"replay {rep}"
        _ = W.wkv_forward(dw, du, dev_f32(k), dev_f32(v))  # unrelated eager work between replays


def test_forward_calls_in_hip_graph_replay_exactly():
    """Several layers of prefill captured once in a HIP graph (as the
    benchmark runs them) give bit-identical outputs and states on every replay,
    with unrelated eager work in between."""
    say("forward graph capture")
    wl = I.WORKLOADS[1].scaled(B=2, T=300, C=96)
    layers = []
    for layer in range(3):
        w, u = I.params(wl, layer)
        k, v = I.kv(wl, layer)
        layers.append((dev_f32(w), dev_f32(u), dev_f32(k), dev_f32(v)))
    calls = [W.ForwardCall(*L) for L in layers]
    for c in calls:
        c()
    torch.cuda.synchronize()
    eager = [(c.out.clone(), c.state_out.clone()) for c in calls]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in calls:
            c()
    for rep in range(3):
        for c in calls:
            c.out.zero_()
            c.state_out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for c, (o, s) in zip(calls, eager):
            assert torch.equal(c.out.view(torch.int32), o.view(torch.int32)), f"replay {rep}"
            assert torch.equal(c.state_out.view(torch.int32), s.view(torch.int32)), f"replay {rep}"
        _ = W.wkv_forward(*layers[0])

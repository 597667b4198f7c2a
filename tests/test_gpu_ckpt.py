"""The training pair wkv_forward_ckpt / wkv_backward_ckpt, through the C
interface.

* The prefill that saves checkpoints gives the same outputs and final state
  as the same kernel without them, bit for bit (sequential and chunked scan,
  gated or not, ragged T around the 8-token chunks and the kernels' tiles).
* The checkpoints are the forward's states: checkpoint j against the float64
  oracle's state after the first 8j tokens, compared representation-free
  (num/den and max_exp + ln den, as final states are), and checkpoint 0 is the
  initial state.
* The backward pass from the checkpoints against the float64 gradient oracle
  (same tolerance as the plain backward): the one-thread-per-lane plan (T <
  64) and the segmented plan (few lanes, T >= 64), with initial and final
  state gradients and with the gate; and against the plain backward on the
  8-layer model's layer shape.
* Argument errors of both entry points.
"""

import ctypes

import numpy as np
import pytest
import torch

from oracle import wkv_backward_direct, wkv_gated_backward_direct, wkv_recurrent
from wkvtest import (F32_TOL, I, W, assert_state_close, dev_f32, host64, make_case,
                     random_state, say)

pytestmark = pytest.mark.gpu

GRAD_TOL = 1e-4
WL0, WL3 = I.WORKLOADS[0], I.WORKLOADS[3]


def rms(a):
    a = np.asarray(a, dtype=np.float64)
    return float(np.sqrt(np.mean(a * a))) if a.size else 1.0


def assert_grad_close(got, ref, tol, what, scale=0.0):
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite gradient"
    err = np.abs(got - ref) / (np.abs(ref) + max(rms(ref), scale, 1e-30))
    worst = float(err.max()) if err.size else 0.0
    assert worst <= tol, f"{what}: max normalised error {worst:.3e} > {tol:.1e}"
    return worst


def bits(t):
    return t.contiguous().view(torch.int32)


FWD_SHAPES = [(1, 1, 8), (2, 7, 33), (2, 8, 16), (2, 9, 40), (2, 63, 24), (1, 257, 32),
              (3, 1000, 40), (1, 2049, 24)]


@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("path", ["seq", "chunk"])
@pytest.mark.parametrize("B,T,C", FWD_SHAPES)
def test_forward_ckpt_outputs_equal_plain_forward(B, T, C, path, gated):
    say(f"forward_ckpt path={path} gated={gated} B={B} T={T} C={C}")
    w, u, k, v = (dev_f32(a) for a in make_case(WL3, B, T, C))
    s0 = dev_f32(random_state(B, C, 7))
    r = dev_f32(I.receptance(WL3.scaled(B=B, T=T, C=C))) if gated else None
    out, st, ck = W.wkv_forward_ckpt(w, u, k, v, r, s0, path=path)
    if gated:
        ref, rst = W.wkv_forward_gated(w, u, k, v, r, s0, path=path)
    else:
        ref, rst = W.wkv_forward_ex(w, u, k, v, s0, path=path)
    torch.cuda.synchronize()
    assert torch.equal(bits(out), bits(ref))
    assert torch.equal(bits(st), bits(rst))
    assert ck.shape == W.ckpt_shape(B, T, C)


@pytest.mark.parametrize("path", ["seq", "chunk"])
@pytest.mark.parametrize("with_state", [False, True])
def test_checkpoints_are_the_forward_states(path, with_state):
    B, T, C = 2, 100, 24
    say(f"checkpoints vs oracle path={path} state={with_state}")
    w, u, k, v = make_case(WL3, B, T, C)
    s0 = random_state(B, C, 8) if with_state else None
    _, _, ck = W.wkv_forward_ckpt(dev_f32(w), dev_f32(u), dev_f32(k), dev_f32(v), None,
                                  None if s0 is None else dev_f32(s0), path=path)
    torch.cuda.synchronize()
    ck = host64(ck)  # (ceil(T/8), B, C, 4): num, den, base, age
    wd = w.astype(np.float64)
    if s0 is None:
        assert np.all(ck[0, ..., 0] == 0) and np.all(ck[0, ..., 1] == 0)
    else:
        assert np.array_equal(ck[0, ..., :3], s0.astype(np.float64).transpose(1, 2, 0))
        assert np.all(ck[0, ..., 3] == 0)
    for j in range(1, ck.shape[0]):
        _, ref = wkv_recurrent(w, u, k[:, :8 * j], v[:, :8 * j], s0)
        got = np.stack([ck[j, ..., 0], ck[j, ..., 1], ck[j, ..., 2] - ck[j, ..., 3] * wd])
        assert_state_close(got, ref, F32_TOL, f"checkpoint {j}")


def gpu_backward_ckpt(w, u, k, v, gout, state_in=None, with_gstate=False, r=None, seed=0):
    dev = lambda a: None if a is None else dev_f32(a)
    dw, du, dk, dv, ds, dr = dev(w), dev(u), dev(k), dev(v), dev(state_in), dev(r)
    _, st, ck = W.wkv_forward_ckpt(dw, du, dk, dv, dr, ds)
    gs_out = None
    if with_gstate:
        g = np.random.default_rng([56, seed])
        shp = (k.shape[0], k.shape[2])
        gs_out = np.stack([g.normal(0, 1, shp), g.normal(0, 1, shp), np.zeros(shp)])
    res = W.wkv_backward(dw, du, dk, dv, dev_f32(gout), ds, st if with_gstate else None,
                         dev(gs_out), r=dr, ckpt=ck)
    torch.cuda.synchronize()
    return [host64(x) for x in res], host64(st), gs_out


def check_ckpt(w, u, k, v, gout, state_in=None, with_gstate=False, r=None, tol=GRAD_TOL):
    got, st, gs_out = gpu_backward_ckpt(w, u, k, v, gout, state_in, with_gstate, r)
    # the oracle takes the final-state gradient at the kernel's final state
    if r is None:
        ref = wkv_backward_direct(w, u, k, v, gout, state_in, gs_out,
                                  st if with_gstate else None)
        names = ("gw", "gu", "gk", "gv", "gstate_in")
        companion = {"gw": 1, "gu": 0, "gk": 3, "gv": 2, "gstate_in": 3}
    else:
        ref = wkv_gated_backward_direct(w, u, k, v, r, gout, state_in, gs_out,
                                        st if with_gstate else None)
        names = ("gw", "gu", "gk", "gv", "gstate_in", "gr")
        companion = {"gw": 1, "gu": 0, "gk": 3, "gv": 2, "gstate_in": 3, "gr": 5}
    errs = {}
    for name, g, rf in zip(names, got, ref):
        if name == "gstate_in" and state_in is None:
            assert np.all(g == 0)
            continue
        errs[name] = assert_grad_close(g, rf, tol, name, rms(ref[companion[name]]))
    return errs


# T < 64 runs the one-thread-per-lane kernel. T >= 64 with few lanes: the
# segmented kernels while B * ceil(C / 32) stays below three quarters of the
# CUs (192 on MI355X), the one-pass chunked kernel from there on (tiles of
# 128 tokens, 32 channels per workgroup). Both with a partial last tile, T
# not a multiple of 8, tile-exact T, idle channel threads (C = 24, 70) and
# several tiles.
BWD_SHAPES = [(1, 1, 8), (2, 7, 33), (2, 45, 24), (2, 150, 24), (1, 300, 32), (2, 1000, 16),
              (2, 256, 40), (1, 136, 70), (1, 1500, 8),
              (192, 150, 24), (96, 136, 70), (192, 256, 32), (200, 400, 8)]


@pytest.mark.parametrize("B,T,C", BWD_SHAPES)
@pytest.mark.parametrize("wl", [WL0, WL3], ids=["dist0", "dist3"])
def test_backward_ckpt_matches_oracle(B, T, C, wl):
    say(f"backward_ckpt B={B} T={T} C={C} wl={wl.wid}")
    w, u, k, v = make_case(wl, B, T, C)
    gout = np.random.default_rng([45, B, T, C]).normal(0, 1, (B, T, C)).astype(np.float32)
    errs = check_ckpt(w, u, k, v, gout)
    say("  " + " ".join(f"{n}={e:.1e}" for n, e in errs.items()))


@pytest.mark.parametrize("B,T", [(2, 45), (2, 150), (192, 150)])
@pytest.mark.parametrize("gated", [False, True])
def test_backward_ckpt_with_states_and_gate(B, T, gated):
    C = 24
    say(f"backward_ckpt states and gate B={B} T={T} gated={gated}")
    w, u, k, v = make_case(WL3, B, T, C)
    gout = np.random.default_rng([46, T]).normal(0, 1, (B, T, C)).astype(np.float32)
    r = I.receptance(WL3.scaled(B=B, T=T, C=C), 1) if gated else None
    s0 = random_state(B, C, 9)
    errs = check_ckpt(w, u, k, v, gout, s0, True, r)
    say("  " + " ".join(f"{n}={e:.1e}" for n, e in errs.items()))


def test_backward_ckpt_agrees_with_plain_backward_on_layer_shape():
    """B=8 T=1024 C=768 (the 8-layer model's layer, segmented plan): the
    gradients from the forward's checkpoints against those of the backward
    that rebuilds its own, to the oracle tolerance (the two start their
    segments from states computed in different orders)."""
    wl = I.WORKLOADS[1]
    say(f"backward_ckpt vs backward B={wl.B} T={wl.T} C={wl.C}")
    w, u = (dev_f32(a) for a in I.params(wl))
    k, v = (dev_f32(a) for a in I.kv(wl))
    gout = dev_f32(I.grad_out(wl))
    _, _, ck = W.wkv_forward_ckpt(w, u, k, v)
    a = W.wkv_backward(w, u, k, v, gout, ckpt=ck)
    b = W.wkv_backward(w, u, k, v, gout)
    torch.cuda.synchronize()
    a = [host64(x) for x in a[:4]]
    b = [host64(x) for x in b[:4]]
    companion = {0: 1, 1: 0, 2: 3, 3: 2}
    for i, name in enumerate(("gw", "gu", "gk", "gv")):
        assert_grad_close(a[i], b[i], GRAD_TOL, name, rms(b[companion[i]]))


def test_ckpt_pair_deterministic_and_in_hip_graph():
    """The checkpoint pair on the 8-layer model's layer shape (one-pass
    backward) and on B=2 T=300 C=40 (segmented): two eager runs agree bit for
    bit (fixed summation orders), and the pair captured once in a HIP graph
    reproduces them on every replay, with the outputs cleared and unrelated
    eager work in between (the workspace needs no clearing between calls)."""
    for B, T, C in ((8, 1024, 768), (2, 300, 40)):
        say(f"checkpoint pair determinism and graph B={B} T={T} C={C}")
        wl = I.WORKLOADS[1].scaled(B=B, T=T, C=C)
        w, u = (dev_f32(a) for a in I.params(wl))
        k, v = (dev_f32(a) for a in I.kv(wl))
        gout = dev_f32(I.grad_out(wl))
        out, st = torch.empty_like(k), torch.empty((3, B, C), device="cuda")
        ck = torch.empty(W.ckpt_shape(B, T, C), device="cuda")
        gk, gv = torch.empty_like(k), torch.empty_like(k)
        gw, gu = torch.empty_like(w), torch.empty_like(w)
        ws = torch.empty(max(W.wkv_backward_workspace_size(B, T, C), 1), dtype=torch.uint8,
                         device="cuda")
        results = (out, st, ck, gk, gv, gw, gu)

        def run():
            W.wkv_forward_ckpt(w, u, k, v, out=out, state_out=st, ckpt=ck)
            W.wkv_backward(w, u, k, v, gout, want_gstate_in=False, workspace=ws,
                           out=(gk, gv, gw, gu, None), ckpt=ck)

        run()
        torch.cuda.synchronize()
        first = [t.clone() for t in results]
        run()
        torch.cuda.synchronize()
        for got, ref in zip(results, first):
            assert torch.equal(got.view(torch.int32), ref.view(torch.int32)), "eager rerun"
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run()
        for rep in range(3):
            for t in results:
                t.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for got, ref in zip(results, first):
                assert torch.equal(got.view(torch.int32), ref.view(torch.int32)), f"replay {rep}"
            _ = W.wkv_backward(w, u, k, v, gout)  # unrelated eager work


def test_ckpt_abi_errors():
    say("checkpoint abi errors")
    lib = W.load_library()
    B, T, C = 2, 20, 8
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    z = lambda *s: torch.zeros(s, device="cuda")
    w, u, k, v, out = z(C), z(C), z(B, T, C), z(B, T, C), z(B, T, C)
    ck = z(*W.ckpt_shape(B, T, C))
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert lib.wkv_ckpt_bytes(B, T, C) == ck.numel() * 4
    # B, T, C, w, u, k, v, r, state_in, out, state_out, ckpt, path, stream
    fwd = [B, T, C, P(w), P(u), P(k), P(v), None, None, P(out), None, P(ck)]
    assert lib.wkv_forward_ckpt(*fwd, W.WKV_PATH_AUTO, s) == 0
    assert lib.wkv_forward_ckpt(*fwd, W.WKV_PATH_LOOKBACK, s) == 7      # no look-back checkpoints
    bad = list(fwd)
    bad[11] = None
    assert lib.wkv_forward_ckpt(*bad, W.WKV_PATH_AUTO, s) == 1          # ckpt missing
    bad[11] = ctypes.c_void_p(ck.data_ptr() + 4)
    assert lib.wkv_forward_ckpt(*bad, W.WKV_PATH_AUTO, s) == 3          # ckpt not 16-byte aligned
    bad[11] = P(out)
    assert lib.wkv_forward_ckpt(*bad, W.WKV_PATH_AUTO, s) == 4          # ckpt on top of out
    gk, gv, gw, gu, g = z(B, T, C), z(B, T, C), z(C), z(C), z(B, T, C)
    need = lib.wkv_backward_workspace_size(B, T, C)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device="cuda")
    # B, T, C, w, u, k, v, r, state_in, state_out, gstate_out, gout, ckpt, gk, gv, gr, gw, gu,
    # gstate_in
    bwd = [B, T, C, P(w), P(u), P(k), P(v), None, None, None, None, P(g), P(ck), P(gk), P(gv),
           None, P(gw), P(gu), None]
    assert lib.wkv_backward_ckpt(*bwd, P(ws), need, s) == 0
    bad = list(bwd)
    bad[12] = None
    assert lib.wkv_backward_ckpt(*bad, P(ws), need, s) == 1             # ckpt missing
    bad[12] = ctypes.c_void_p(ck.data_ptr() + 8)
    assert lib.wkv_backward_ckpt(*bad, P(ws), need, s) == 3             # not 16-byte aligned
    bad[12] = P(gk)
    assert lib.wkv_backward_ckpt(*bad, P(ws), need, s) == 4             # an output on top of it
    torch.cuda.synchronize()

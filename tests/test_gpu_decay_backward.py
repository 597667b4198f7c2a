"""GPU parity of the per-token-decay backward (wkv_backward_dd) with its
float64 oracle (oracle/wkv_grad.py, wkv_dd_backward_direct, pinned in
test_oracle_grad_decay.py), through the C interface: the one-thread-per-lane
plan (T < 64, or B*C >= 2^16) and the segmented one (few lanes, T >= 64) on
ragged sizes, with initial states and a final-state gradient, extreme keys,
a state-wiping rate, the empty cases, and, at the 8-layer model's layer
shape, the constant-rate case against the constant-decay backward.

Tolerance: 1e-4 of each element (or of the gradient's typical size where the
element is near zero), as for the constant-decay backward."""

import numpy as np
import pytest
import torch

from oracle import wkv_dd_backward_direct, wkv_dd_recurrent
from wkvtest import (I, W, assert_grad_close, assert_state_close, dev_f32, host64, make_case,
                     random_state, rms,
                     say)

pytestmark = pytest.mark.gpu

GRAD_TOL = 1e-4
WL0, WL3 = I.WORKLOADS[0], I.WORKLOADS[3]


def dd_case(wl, B, T, C, layer=0):
    w, u, k, v = make_case(wl, B, T, C, layer)
    wt = I.decay_rates(wl.scaled(B=B, T=T, C=C), layer)
    g = np.random.default_rng([61, B, T, C, layer]).normal(0, 1, (B, T, C)).astype(np.float32)
    return wt, u, k, v, g


def check(wt, u, k, v, gout, state_in=None, with_gstate=False, tol=GRAD_TOL):
    dev = lambda a: None if a is None else dev_f32(a)
    st_out = gs_out = None
    if with_gstate:
        _, st = W.wkv_forward_dd(dev(wt), dev(u), dev(k), dev(v), dev(state_in))
        st_out = host64(st)
        g = np.random.default_rng([62, k.shape[1]])
        shp = (k.shape[0], k.shape[2])
        gs_out = np.stack([g.normal(0, 1, shp), g.normal(0, 1, shp), np.zeros(shp)])
    got = W.wkv_backward_dd(dev(wt), dev(u), dev(k), dev(v), dev(gout), dev(state_in),
                            dev(st_out), dev(gs_out))
    torch.cuda.synchronize()
    got = [host64(x) for x in got]
    ref = wkv_dd_backward_direct(wt, u, k, v, gout, state_in, gs_out, st_out)
    names = ("gw", "gu", "gk", "gv", "gstate_in")
    errs = {}
    for i, name in enumerate(names):
        if name == "gstate_in" and state_in is None:
            assert np.all(got[i] == 0)
            continue
        scale = rms(ref[3]) if name in ("gk", "gw") else 0.0
        errs[name] = assert_grad_close(got[i], ref[i], tol, name, scale)
    return errs


# T < 64: one thread per lane; T >= 64 with these few lanes: segmented
SHAPES = [(1, 1, 8), (2, 7, 33), (2, 45, 24), (1, 63, 16), (2, 150, 24), (1, 300, 32),
          (2, 777, 16), (1, 1500, 8)]


@pytest.mark.parametrize("B,T,C", SHAPES)
@pytest.mark.parametrize("wl", [WL0, WL3], ids=["dist0", "dist3"])
def test_dd_backward_matches_oracle(B, T, C, wl):
    say(f"dd backward B={B} T={T} C={C} wl={wl.wid}")
    errs = check(*dd_case(wl, B, T, C))
    say("  " + " ".join(f"{n}={e:.1e}" for n, e in errs.items()))


@pytest.mark.parametrize("T", [45, 150])
def test_dd_backward_with_states(T):
    B, C = 2, 24
    say(f"dd backward states T={T}")
    wt, u, k, v, g = dd_case(WL3, B, T, C, 1)
    errs = check(wt, u, k, v, g, random_state(B, C, 11), True)
    say("  " + " ".join(f"{n}={e:.1e}" for n, e in errs.items()))


def test_dd_backward_many_lanes():
    """B*C >= 2^16 with T >= 64: the one-thread-per-lane plan past its first
    checkpoint chunks."""
    B, T, C = 86, 72, 768
    say(f"dd backward B={B} T={T} C={C}")
    errs = check(*dd_case(WL0, B, T, C))
    say("  " + " ".join(f"{n}={e:.1e}" for n, e in errs.items()))


def test_dd_backward_state_wiping_rate():
    """A huge rate in the middle of the sequence decays every earlier term
    to nothing: the gradients of the tokens before it vanish for the outputs
    after it, and nothing overflows."""
    B, T, C = 2, 150, 16
    wt, u, k, v, g = dd_case(WL0, B, T, C, 2)
    wt[:, 70] = 1e4
    errs = check(wt, u, k, v, g, random_state(B, C, 12), True)
    say("  " + " ".join(f"{n}={e:.1e}" for n, e in errs.items()))


def test_dd_backward_empty_cases():
    """T = 0: the initial state's gradient is the final state's, passed
    through; B = 0: dL/du is zero."""
    C = 8
    for B, T in ((2, 0), (0, 5)):
        say(f"dd backward empty B={B} T={T}")
        z = lambda *s: torch.zeros(s, device="cuda")
        s0 = dev_f32(random_state(B, C, 13)) if B else None
        gs = dev_f32(random_state(B, C, 14)) if B else None
        st = s0
        gw, gu, gk, gv, gsi = W.wkv_backward_dd(z(B, T, C), z(C), z(B, T, C), z(B, T, C),
                                                z(B, T, C), s0, st, gs)
        torch.cuda.synchronize()
        assert torch.all(gu == 0)
        if B:
            ref = host64(gs)
            gsi = host64(gsi)
            assert np.allclose(gsi[:2], ref[:2], rtol=1e-6, atol=0)
            s0h = host64(s0)
            assert np.allclose(gsi[2], s0h[0] * ref[0] + s0h[1] * ref[1], rtol=1e-5, atol=1e-6)


def test_dd_backward_constant_rate_equals_constant_decay_backward():
    """At B=8 T=1024 C=768 (the 8-layer model's layer): with every rate equal
    to the channel's w the gradients are the constant-decay backward's, the
    rate gradients summed over batch rows and positions giving dL/dw."""
    wl = I.WORKLOADS[1]
    say(f"dd backward constant rate vs backward B={wl.B} T={wl.T} C={wl.C}")
    w, u = (dev_f32(a) for a in I.params(wl))
    k, v = (dev_f32(a) for a in I.kv(wl))
    g = dev_f32(I.grad_out(wl))
    wt = w.expand(wl.B, wl.T, wl.C).contiguous()
    a = W.wkv_backward_dd(wt, u, k, v, g)
    b = W.wkv_backward(w, u, k, v, g)
    torch.cuda.synchronize()
    gw_sum = a[0].double().sum(dim=(0, 1)).cpu().numpy()
    assert_grad_close(gw_sum, host64(b[0]), GRAD_TOL, "gw", rms(host64(b[1])))
    for i, name in ((1, "gu"), (2, "gk"), (3, "gv")):
        assert_grad_close(host64(a[i]), host64(b[i]), GRAD_TOL, name)


def test_dd_backward_deterministic_and_in_hip_graph():
    """Two eager calls agree bit for bit (fixed summation orders), and a call
    captured in a HIP graph reproduces them on every replay, with the outputs
    cleared and unrelated eager work in between; the segmented plan (B=8
    T=1024 C=768) and the one-thread-per-lane plan (B=90 T=40 C=768)."""
    for B, T, C in ((8, 1024, 768), (90, 40, 768)):
        say(f"dd backward determinism and graph B={B} T={T} C={C}")
        wt, u, k, v, g = (dev_f32(a) for a in dd_case(WL0, B, T, C))
        s0 = dev_f32(random_state(B, C, 15))
        outs = (torch.empty_like(k), torch.empty_like(k), torch.empty_like(k),
                torch.empty_like(u), torch.empty((3, B, C), device="cuda"))
        ws = torch.empty(max(W.wkv_backward_dd_workspace_size(B, T, C), 1), dtype=torch.uint8,
                         device="cuda")

        def run():
            W.wkv_backward_dd(wt, u, k, v, g, s0, workspace=ws, out=outs)

        run()
        torch.cuda.synchronize()
        first = [t.clone() for t in outs]
        run()
        torch.cuda.synchronize()
        bits = lambda t: t.view(torch.int32)
        for got, ref in zip(outs, first):
            assert torch.equal(bits(got), bits(ref)), "eager rerun"
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run()
        for rep in range(3):
            for t in outs:
                t.zero_()
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            for got, ref in zip(outs, first):
                assert torch.equal(bits(got), bits(ref)), f"replay {rep}"
            _ = W.wkv_backward_dd(wt, u, k, v, g)  # unrelated eager work


# ---------------------------------------------------------------- checkpoints

CK_SHAPES = [(1, 1, 8), (2, 7, 33), (2, 63, 24), (1, 257, 32), (2, 300, 40), (1, 2100, 16)]


def ck_records(ck):
    """(num, den, max_exp) planes of wkv_forward_dd_ckpt's 16-byte records:
    two float32 values, then a float64."""
    ck = ck.contiguous()
    nd = host64(ck[..., :2])
    m = ck.view(torch.float64)[..., 1].double().cpu().numpy()
    return nd[..., 0], nd[..., 1], m


@pytest.mark.parametrize("path", ["seq", "chunk"])
@pytest.mark.parametrize("B,T,C", CK_SHAPES)
def test_dd_forward_ckpt_outputs_equal_plain_forward(B, T, C, path):
    say(f"dd forward_ckpt vs forward path={path} B={B} T={T} C={C}")
    wt, u, k, v, _ = (dev_f32(a) for a in dd_case(WL3, B, T, C))
    s0 = dev_f32(random_state(B, C, 16))
    out, st, ck = W.wkv_forward_dd_ckpt(wt, u, k, v, s0, path=path)
    ref, rst = W.wkv_forward_dd(wt, u, k, v, s0, path=path)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32), ref.view(torch.int32))
    assert torch.equal(st.view(torch.int32), rst.view(torch.int32))


@pytest.mark.parametrize("path", ["seq", "chunk"])
def test_dd_checkpoints_are_the_forward_states(path):
    """Record j holds the state in front of token 8j: the oracle's state after
    the first 8j tokens (the initial state for j = 0)."""
    B, T, C = 2, 150, 40
    say(f"dd checkpoints vs oracle states path={path}")
    wt, u, k, v, _ = dd_case(WL0, B, T, C)
    s0 = random_state(B, C, 17)
    _, _, ck = W.wkv_forward_dd_ckpt(dev_f32(wt), dev_f32(u), dev_f32(k), dev_f32(v),
                                     dev_f32(s0), path=path)
    torch.cuda.synchronize()
    n, d, m = ck_records(ck)
    for j in range(n.shape[0]):
        t = 8 * j
        if t == 0:
            ref = s0.astype(np.float64)
        else:
            _, ref = wkv_dd_recurrent(wt[:, :t], u, k[:, :t], v[:, :t], s0)
        assert_state_close(np.stack([n[j], d[j], m[j]]), ref, 1e-5, f"checkpoint {j}")


@pytest.mark.parametrize("B,T,C", [(2, 45, 24), (2, 150, 24), (1, 300, 32), (2, 777, 16)])
def test_dd_backward_ckpt_matches_oracle(B, T, C):
    say(f"dd backward_ckpt B={B} T={T} C={C}")
    wt, u, k, v, g = dd_case(WL3, B, T, C, 3)
    s0 = random_state(B, C, 18)
    dev = lambda a: None if a is None else dev_f32(a)
    _, st, ck = W.wkv_forward_dd_ckpt(dev(wt), dev(u), dev(k), dev(v), dev(s0))
    st_out = host64(st)
    gen = np.random.default_rng([63, T])
    gs_out = np.stack([gen.normal(0, 1, (B, C)), gen.normal(0, 1, (B, C)), np.zeros((B, C))])
    got = W.wkv_backward_dd(dev(wt), dev(u), dev(k), dev(v), dev(g), dev(s0), st,
                            dev(gs_out), ckpt=ck)
    torch.cuda.synchronize()
    got = [host64(x) for x in got]
    ref = wkv_dd_backward_direct(wt, u, k, v, g, s0, gs_out, st_out)
    for i, name in enumerate(("gw", "gu", "gk", "gv", "gstate_in")):
        scale = rms(ref[3]) if name in ("gk", "gw") else 0.0
        assert_grad_close(got[i], ref[i], GRAD_TOL, name, scale)


@pytest.mark.parametrize("B,T,C", [(8, 1024, 768), (90, 100, 768)])
def test_dd_backward_ckpt_agrees_with_plain_backward(B, T, C):
    """The 8-layer model's layer (segmented plan) and B*C >= 2^16 (one thread
    per lane): gradients from the forward's checkpoints against those of the
    backward that rebuilds its own, to the oracle tolerance."""
    say(f"dd backward_ckpt vs backward B={B} T={T} C={C}")
    wt, u, k, v, g = (dev_f32(a) for a in dd_case(WL0, B, T, C))
    _, _, ck = W.wkv_forward_dd_ckpt(wt, u, k, v)
    a = W.wkv_backward_dd(wt, u, k, v, g, ckpt=ck)
    b = W.wkv_backward_dd(wt, u, k, v, g)
    torch.cuda.synchronize()
    a = [host64(x) for x in a[:4]]
    b = [host64(x) for x in b[:4]]
    for i, name in enumerate(("gw", "gu", "gk", "gv")):
        scale = rms(b[3]) if name in ("gk", "gw") else 0.0
        assert_grad_close(a[i], b[i], GRAD_TOL, name, scale)

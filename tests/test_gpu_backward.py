"""GPU parity of the backward pass (wkv_backward) against the float64 gradient
oracle (oracle/wkv_grad.py, pinned by finite differences in
test_oracle_grad.py).

Tolerance. The gradients are sums over up to T positions of products of
forward quantities that the fp32 kernel knows to ~1e-6 relative, and dL/dk
and dL/dw subtract two such sums. They are compared elementwise with
|got - ref| / (|ref| + s) against 1e-4 (fp32 I/O), s = the RMS of the
reference tensor or of its companion (dL/dv for dL/dk and the state, dL/du
for dL/dw), whichever is larger: dL/dk and dL/dw can be exactly zero (T = 1,
T <= 2) where the kernel's fp32 sums leave a rounding residue of the size of
the other gradients' ulp. Extreme keys widen the bound by the exponent's own
uncertainty, as in the forward tests."""

import ctypes

import numpy as np
import pytest
import torch

from oracle import wkv_backward_direct, wkv_recurrent
from wkvtest import I, W, dev_f32, host64, make_case, random_state, say

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


def gpu_backward(w, u, k, v, gout, state_in=None, state_out=None, gstate_out=None):
    dev = lambda a: None if a is None else dev_f32(a)
    gw, gu, gk, gv, gs = W.wkv_backward(dev(w), dev(u), dev(k), dev(v), dev(gout), dev(state_in),
                                        dev(state_out), dev(gstate_out))
    torch.cuda.synchronize()
    return host64(gw), host64(gu), host64(gk), host64(gv), host64(gs)


def check(w, u, k, v, gout, state_in=None, with_gstate=False, tol=GRAD_TOL, seed=0):
    st_out = gs_out = None
    if with_gstate:
        _, st_out = wkv_recurrent(w, u, k, v, state_in)
        st_out = st_out.astype(np.float32).astype(np.float64)
        g = np.random.default_rng([55, seed])
        gs_out = np.stack([g.normal(0, 1, st_out.shape[1:]), g.normal(0, 1, st_out.shape[1:]),
                           np.zeros(st_out.shape[1:])])
    ref = wkv_backward_direct(w, u, k, v, gout, state_in, gs_out, st_out)
    got = gpu_backward(w, u, k, v, gout, state_in, st_out, gs_out)
    errs = {}
    companion = {"gw": 1, "gu": 0, "gk": 3, "gv": 2, "gstate_in": 3}
    for name, g, r in zip(("gw", "gu", "gk", "gv", "gstate_in"), got, ref):
        if name == "gstate_in" and state_in is None:
            assert np.all(g == 0)
            continue
        errs[name] = assert_grad_close(g, r, tol, name, rms(ref[companion[name]]))
    return errs


SHAPES = [(1, 1, 8), (2, 7, 33), (2, 8, 16), (2, 37, 40), (3, 64, 64), (1, 300, 32)]


@pytest.mark.parametrize("B,T,C", SHAPES)
@pytest.mark.parametrize("wl", [WL0, WL3], ids=["dist0", "dist3"])
def test_backward_matches_oracle(B, T, C, wl):
    say(f"backward B={B} T={T} C={C} wl={wl.wid}")
    w, u, k, v = make_case(wl, B, T, C)
    gout = np.random.default_rng([41, B, T, C]).normal(0, 1, (B, T, C)).astype(np.float32)
    errs = check(w, u, k, v, gout)
    say("  " + " ".join(f"{n}={e:.1e}" for n, e in errs.items()))


@pytest.mark.parametrize("T", [45, 150])
@pytest.mark.parametrize("with_state,with_gstate", [(True, False), (False, True), (True, True)])
def test_backward_with_states(with_state, with_gstate, T):
    """T = 45 runs the one-thread-per-lane kernel, T = 150 (few lanes) the
    segmented kernels, whose segments are chained both ways."""
    B, C = 2, 24
    say(f"backward states in={with_state} out={with_gstate} T={T}")
    w, u, k, v = make_case(WL3, B, T, C)
    gout = np.random.default_rng([42]).normal(0, 1, (B, T, C)).astype(np.float32)
    s0 = random_state(B, C, 3) if with_state else None
    errs = check(w, u, k, v, gout, s0, with_gstate)
    say("  " + " ".join(f"{n}={e:.1e}" for n, e in errs.items()))


def test_backward_empty_sequence_passes_state_gradient():
    """T = 0: the final state is the initial one, so its gradient goes straight
    through (rescaled between the two max_exp values) and dL/dw = dL/du = 0."""
    B, C = 2, 16
    say("backward T=0")
    w, u, k, v = make_case(WL0, B, 1, C)
    k, v = k[:, :0], v[:, :0]
    s0 = random_state(B, C, 4)
    gout = np.zeros((B, 0, C), np.float32)
    errs = check(w, u, k, v, gout, s0, True)
    say("  " + " ".join(f"{n}={e:.1e}" for n, e in errs.items()))


@pytest.mark.parametrize("kmag", [60.0, 1e4])
def test_backward_extreme_keys(kmag):
    B, T, C = 2, 200, 32
    say(f"backward extreme keys k=+-{kmag}")
    w, u, _, v = make_case(WL3, B, T, C)
    g = np.random.default_rng([8, int(kmag)])
    k = g.choice(np.array([-kmag, kmag, 0.0, 1.0, -3.0], dtype=np.float32), size=(B, T, C))
    gout = g.normal(0, 1, (B, T, C)).astype(np.float32)
    tol = max(GRAD_TOL, 8 * float(np.spacing(np.float32(kmag))))
    check(w, u, k, v, gout, tol=tol)


def test_backward_deterministic():
    B, T, C = 4, 129, 48
    say("backward determinism")
    w, u, k, v = make_case(WL3, B, T, C)
    gout = np.random.default_rng([43]).normal(0, 1, (B, T, C)).astype(np.float32)
    a = gpu_backward(w, u, k, v, gout)
    b = gpu_backward(w, u, k, v, gout)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_backward_large_batch_sampled_channels():
    """The decode workload's prefill shape (B=256, T=512) on 4 channels: every
    batch row, so dL/dw and dL/du (sums over the batch) are checked too."""
    wl = I.WORKLOADS[2]
    B, T, C = wl.B, wl.T, 4
    say(f"backward B={B} T={T} C={C}")
    w, u, k, v = make_case(wl, B, T, C)
    gout = np.random.default_rng([44]).normal(0, 1, (B, T, C)).astype(np.float32)
    errs = check(w, u, k, v, gout)
    say("  " + " ".join(f"{n}={e:.1e}" for n, e in errs.items()))


@pytest.mark.parametrize("wid,chans", [(1, (0, 31, 32, 300, 511, 767)), (2, (0, 385, 767))],
                         ids=["B8_T1024_C768", "B256_T512_C768"])
@pytest.mark.parametrize("ckpt", [False, True], ids=["plain", "from_checkpoints"])
def test_backward_at_benchmark_shapes_on_sampled_channels(wid, chans, ckpt):
    """The two benchmarked backward shapes (one layer of the 8-layer model:
    B=8 T=1024 C=768, the segmented or one-pass chunked plan; B=256 T=512
    C=768, one thread per lane) run at full size, through the plain backward
    and the one from the forward's checkpoints; the oracle checks every batch
    row of a few channels (group edges included), so dL/dw and dL/du, sums
    over the batch, are checked too."""
    wl = I.WORKLOADS[wid].scaled(decode_steps=0)
    say(f"backward at B={wl.B} T={wl.T} C={wl.C} ckpt={ckpt}, channels {chans}")
    w, u = I.params(wl)
    k, v = I.kv(wl)
    gout = I.grad_out(wl)
    dw, du, dk, dv, dg = (dev_f32(a) for a in (w, u, k, v, gout))
    ck = W.wkv_forward_ckpt(dw, du, dk, dv)[2] if ckpt else None
    got = W.wkv_backward(dw, du, dk, dv, dg, ckpt=ck)
    torch.cuda.synchronize()
    cs = list(chans)
    got = [host64(x) for x in got[:4]]
    got = [got[0][cs], got[1][cs], got[2][:, :, cs], got[3][:, :, cs]]
    ref = wkv_backward_direct(w[cs], u[cs], k[:, :, cs], v[:, :, cs], gout[:, :, cs])
    companion = {0: 1, 1: 0, 2: 3, 3: 2}
    errs = {}
    for i, name in enumerate(("gw", "gu", "gk", "gv")):
        errs[name] = assert_grad_close(got[i], ref[i], GRAD_TOL, name, rms(ref[companion[i]]))
    say("  " + " ".join(f"{n}={e:.1e}" for n, e in errs.items()))


def test_backward_abi_errors():
    say("backward abi errors")
    lib = W.load_library()
    B, T, C = 2, 20, 8
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    z = lambda *s: torch.zeros(s, device="cuda")
    w, u, k, v, g = z(C), z(C), z(B, T, C), z(B, T, C), z(B, T, C)
    gk, gv, gw, gu = z(B, T, C), z(B, T, C), z(C), z(C)
    need = lib.wkv_backward_workspace_size(B, T, C)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    # B, T, C, w, u, k, v, r, state_in, state_out, gstate_out, gout, gk, gv, gr, gw, gu, gstate_in
    base = [B, T, C, P(w), P(u), P(k), P(v), None, None, None, None, P(g), P(gk), P(gv), None,
            P(gw), P(gu), None]
    assert lib.wkv_backward(*base, P(ws), need, s) == 0
    assert lib.wkv_backward(*base, P(ws), need - 16, s) == 8            # workspace too small
    bad = list(base)
    bad[9] = P(z(3, B, C))                                              # state_out without gradient
    assert lib.wkv_backward(*bad, P(ws), need, s) == 1
    bad = list(base)
    bad[7] = P(z(B, T, C))                                              # r without dL/dr
    assert lib.wkv_backward(*bad, P(ws), need, s) == 1
    bad = list(base)
    bad[12] = P(k)                                                      # gk on top of k
    assert lib.wkv_backward(*bad, P(ws), need, s) == 4
    bad = list(base)
    bad[0] = 0                                                          # B = 0: gw, gu zeroed
    gw.fill_(5.0)
    assert lib.wkv_backward(*bad, None, 0, s) == 0
    torch.cuda.synchronize()
    assert torch.all(gw == 0) and torch.all(gu == 0)

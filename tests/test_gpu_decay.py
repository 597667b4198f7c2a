"""GPU parity of the per-token-decay operator (wkv_forward_dd, wkv_step_dd)
with its float64 oracle (oracle/wkv_decay.py, pinned in
test_oracle_decay.py), through the C interface: ragged sizes around both
kernels' tiles, initial and in-place states, split/resume, decode steps,
bf16 I/O, extreme keys, a state-wiping rate, the constant-rate case against
the constant-decay kernels, the error paths and a sampled check at the
8-layer model's layer shape.

Tolerances are those of the constant-decay kernels (wkvtest): 1e-5 for fp32,
2e-2 for bf16 I/O, extreme keys included."""

import ctypes

import numpy as np
import pytest
import torch

from oracle import wkv_dd_recurrent, wkv_dd_step_ref
from wkvtest import (BF16_TOL, F32_TOL, I, W, assert_out_close, assert_state_close, dev_f32,
                     dev_io, host64, make_case, random_state, say, tol_for)

pytestmark = pytest.mark.gpu

PATHS = ["seq", "chunk"]
WL0, WL3, WL4 = I.WORKLOADS[0], I.WORKLOADS[3], I.WORKLOADS[4]

# T around the chunked kernel's tiles (64 tokens up to T = 256, then 128 for
# fp32 and 64 for paired bf16, with a change of workgroup shape at T = 2048)
# and C around its 32-channel groups.
SHAPES = [
    (1, 1, 1), (2, 2, 7), (3, 31, 33), (2, 63, 48), (2, 64, 64), (2, 65, 17), (1, 255, 16),
    (1, 256, 32), (1, 257, 80), (1, 384, 40), (2, 511, 24), (2, 640, 24), (1, 1000, 40),
    (1, 2048, 8), (1, 2049, 96), (2, 3000, 100), (1, 4097, 16),
]


def dd_case(wl, B, T, C, layer=0):
    w, u, k, v = make_case(wl, B, T, C, layer)
    wt = I.decay_rates(wl.scaled(B=B, T=T, C=C), layer)
    return wt, u, k, v


def gpu_dd(wt, u, k, v, io="f32", state_in=None, path="auto"):
    ds = None if state_in is None else dev_f32(state_in)
    out, st = W.wkv_forward_dd(dev_io(wt, io), dev_f32(u), dev_io(k, io), dev_io(v, io), ds,
                               path=path)
    torch.cuda.synchronize()
    return host64(out), host64(st)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("B,T,C", SHAPES)
@pytest.mark.parametrize("wl", [WL0, WL3], ids=["dist0", "dist3"])
def test_dd_forward_f32(path, B, T, C, wl):
    say(f"dd forward f32 path={path} B={B} T={T} C={C} wl={wl.wid}")
    wt, u, k, v = dd_case(wl, B, T, C)
    got, gst = gpu_dd(wt, u, k, v, "f32", path=path)
    ref, rst = wkv_dd_recurrent(wt, u, k, v)
    assert_out_close(got, ref, v, F32_TOL)
    assert_state_close(gst, rst, F32_TOL)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("B,T,C", [(1, 1, 2), (2, 3, 6), (2, 65, 34), (1, 257, 64),
                                   (3, 700, 32), (1, 2049, 66), (1, 130, 7), (1, 2500, 130),
                                   (64, 300, 256), (1, 5, 512), (1, 16, 512), (3, 24, 1536)])
def test_dd_forward_bf16(path, B, T, C):
    say(f"dd forward bf16 path={path} B={B} T={T} C={C}")
    wt, u, k, v = dd_case(WL4, B, T, C)
    got, gst = gpu_dd(wt, u, k, v, "bf16", path=path)
    ref, rst = wkv_dd_recurrent(wt, u, k, v)
    assert_out_close(got, ref, v, BF16_TOL)
    assert_state_close(gst, rst, F32_TOL * 10)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_dd_forward_from_initial_state(path, io):
    B, T, C = 2, 300, 48
    say(f"dd initial state path={path} io={io}")
    wt, u, k, v = dd_case(WL4 if io == "bf16" else WL3, B, T, C)
    s0 = random_state(B, C, 11)
    got, gst = gpu_dd(wt, u, k, v, io, state_in=s0, path=path)
    ref, rst = wkv_dd_recurrent(wt, u, k, v, s0.astype(np.float64))
    assert_out_close(got, ref, v, tol_for(io))
    assert_state_close(gst, rst, F32_TOL * (10 if io == "bf16" else 1))


def test_dd_bf16_sequential_scan_both_widths_from_state():
    """The bf16 sequential scan from an initial state at a wide row (C = 1024,
    T = 333 ends in a partial block of the walk's 8-token unroll): first with
    aligned buffers (two channels per thread), then with the same values one
    element off 4-byte alignment (one channel per thread), to the same
    result."""
    B, T, C = 2, 333, 1024
    say("dd bf16 sequential scan, both widths, from state")
    wt, u, k, v = dd_case(WL4, B, T, C)
    s0 = random_state(B, C, 5)
    got, gst = gpu_dd(wt, u, k, v, "bf16", state_in=s0, path="seq")
    ref, rst = wkv_dd_recurrent(wt, u, k, v, s0.astype(np.float64))
    assert_out_close(got, ref, v, BF16_TOL)
    assert_state_close(gst, rst, F32_TOL * 10)

    def off(x):  # the same values at a 2-byte offset inside a larger buffer
        flat = torch.empty(x.size + 1, dtype=torch.bfloat16, device="cuda")
        flat[1:] = dev_io(x, "bf16").reshape(-1)
        return flat[1:].view(x.shape)
    out = torch.empty(B * T * C + 1, dtype=torch.bfloat16, device="cuda")[1:].view(B, T, C)
    o2, st2 = W.wkv_forward_dd(off(wt), dev_f32(u), off(k), off(v), dev_f32(s0), out=out,
                               path="seq")
    torch.cuda.synchronize()
    assert_out_close(host64(o2), ref, v, BF16_TOL)
    assert_state_close(host64(st2), rst, F32_TOL * 10)


@pytest.mark.parametrize("path", PATHS)
def test_dd_state_in_place_and_split_resume(path):
    B, T, C = 2, 333, 40
    say(f"dd in-place state and split path={path}")
    wt, u, k, v = dd_case(WL3, B, T, C)
    ref, rst = wkv_dd_recurrent(wt, u, k, v)
    ds = dev_f32(np.stack([np.zeros((B, C)), np.zeros((B, C)), np.full((B, C), -1e38)]))
    outs = []
    for lo, hi in ((0, 100), (100, 101), (101, T)):
        o, _ = W.wkv_forward_dd(dev_f32(wt[:, lo:hi]), dev_f32(u), dev_f32(k[:, lo:hi]),
                                dev_f32(v[:, lo:hi]), ds, state_out=ds, path=path)
        outs.append(o)
    torch.cuda.synchronize()
    got = np.concatenate([host64(o) for o in outs], axis=1)
    assert_out_close(got, ref, v, F32_TOL)
    assert_state_close(host64(ds), rst, F32_TOL)


@pytest.mark.parametrize("path", PATHS)
def test_dd_constant_rate_is_the_constant_decay_operator(path):
    """w_t = w for every t: the per-token kernels agree with the constant-decay
    kernels (and both with the oracle)."""
    B, T, C = 2, 700, 64
    say(f"dd constant rate path={path}")
    w, u, k, v = make_case(WL3, B, T, C)
    wt = np.broadcast_to(w, (B, T, C)).copy()
    got, gst = gpu_dd(wt, u, k, v, "f32", path=path)
    base, _ = W.wkv_forward_ex(dev_f32(w), dev_f32(u), dev_f32(k), dev_f32(v), path=path)
    torch.cuda.synchronize()
    ref, rst = wkv_dd_recurrent(wt, u, k, v)
    assert_out_close(got, ref, v, F32_TOL)
    assert_out_close(got, host64(base), v, 2 * F32_TOL, "dd vs constant-decay kernel")
    assert_state_close(gst, rst, F32_TOL)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_dd_step_matches_oracle_and_forward(io):
    """A prefill of 40 tokens, then 12 decode steps with their own rates; the
    steps also equal the prefill of the whole sequence."""
    B, T, C, S = 3, 40, 52, 12
    say(f"dd decode steps io={io}")
    wl = WL4 if io == "bf16" else WL3
    wt, u, k, v = dd_case(wl, B, T + S, C)
    ref, rst = wkv_dd_recurrent(wt, u, k, v)
    _, st = W.wkv_forward_dd(dev_io(wt[:, :T], io), dev_f32(u), dev_io(k[:, :T], io),
                             dev_io(v[:, :T], io))
    outs = []
    for s in range(T, T + S):
        outs.append(W.wkv_step_dd(dev_io(wt[:, s], io), dev_f32(u), dev_io(k[:, s], io),
                                  dev_io(v[:, s], io), st))
    torch.cuda.synchronize()
    got = np.stack([host64(o) for o in outs], axis=1)
    assert_out_close(got, ref[:, T:], v[:, T:], tol_for(io))
    assert_state_close(host64(st), rst, F32_TOL * (10 if io == "bf16" else 1))
    # one step against the oracle's own step from the same state
    s0 = random_state(B, C, 12)
    ds = dev_f32(s0)
    o = W.wkv_step_dd(dev_io(wt[:, 0], io), dev_f32(u), dev_io(k[:, 0], io), dev_io(v[:, 0], io),
                      ds)
    torch.cuda.synchronize()
    ro, rs = wkv_dd_step_ref(wt[:, 0], u, k[:, 0], v[:, 0], s0.astype(np.float64))
    assert_out_close(host64(o), ro, v[:, 0], tol_for(io))
    assert_state_close(host64(ds), rs, F32_TOL)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("kmag", [60.0, 88.0, 1e4])
def test_dd_extreme_keys(path, kmag):
    B, T, C = 2, 400, 40
    say(f"dd extreme keys path={path} k=+-{kmag}")
    g = np.random.default_rng([17, int(kmag)])
    wt, u, _, v = dd_case(WL3, B, T, C)
    k = g.choice(np.array([-kmag, kmag, 0.0, 1.0, -3.0], dtype=np.float32), size=(B, T, C))
    got, gst = gpu_dd(wt, u, k, v, "f32", path=path)
    ref, rst = wkv_dd_recurrent(wt, u, k, v)
    # every exponent difference is formed in fp64 and rounded once, so keys on
    # the coarse fp32 grid of |k| = 1e4 are held to the flat bound (measured on
    # MI355X: 1.2e-7 on both paths)
    e = assert_out_close(got, ref, v, F32_TOL)
    say(f"  max normalised output error {e:.3e} (bound {F32_TOL:.1e})")
    assert_state_close(gst, rst, F32_TOL)


@pytest.mark.parametrize("path", PATHS)
def test_dd_huge_rate_wipes_the_state(path):
    """A rate of 1e4 at step t0 leaves only token t0 in the state: the outputs
    after it equal a fresh run from t0."""
    B, T, C, t0 = 2, 300, 36, 137
    say(f"dd state-wiping rate path={path}")
    wt, u, k, v = dd_case(WL0, B, T, C)
    wt[:, t0] = 1e4
    s0 = random_state(B, C, 13)
    got, _ = gpu_dd(wt, u, k, v, "f32", s0, path=path)
    fresh, _ = gpu_dd(wt[:, t0:], u, k[:, t0:], v[:, t0:], "f32", path=path)
    assert_out_close(got[:, t0 + 1:], fresh[:, 1:], v[:, t0 + 1:], 2 * F32_TOL)
    ref, _ = wkv_dd_recurrent(wt, u, k, v, s0.astype(np.float64))
    assert_out_close(got, ref, v, F32_TOL)


@pytest.mark.parametrize("path", PATHS)
def test_dd_deterministic(path):
    B, T, C = 2, 1500, 72
    say(f"dd determinism path={path}")
    wt, u, k, v = dd_case(WL3, B, T, C)
    a, sa = gpu_dd(wt, u, k, v, "f32", path=path)
    b, sb = gpu_dd(wt, u, k, v, "f32", path=path)
    assert np.array_equal(a, b) and np.array_equal(sa, sb)


def test_dd_empty_and_degenerate_sizes():
    say("dd T=0, B=0, C=0")
    B, C = 2, 24
    s0 = random_state(B, C, 14)
    ds, dso = dev_f32(s0), dev_f32(np.zeros((3, B, C)))
    e = torch.empty((B, 0, C), device="cuda")
    W.wkv_forward_dd(e, dev_f32(np.zeros(C)), e, e, ds, state_out=dso)
    torch.cuda.synchronize()
    assert np.array_equal(host64(dso), s0.astype(np.float64))
    # no state in: the empty state comes out
    W.wkv_forward_dd(e, dev_f32(np.zeros(C)), e, e, None, state_out=dso)
    torch.cuda.synchronize()
    st = host64(dso)
    assert np.all(st[:2] == 0) and np.all(st[2] == np.float32(-1e38))
    for shape in ((0, 5, C), (B, 5, 0)):
        z = torch.zeros(shape, device="cuda")
        out, _ = W.wkv_forward_dd(z, dev_f32(np.zeros(shape[2])), z, z)
        assert out.shape == shape


def test_dd_abi_errors():
    say("dd abi errors")
    lib = W.load_library()
    B, T, C = 2, 20, 8
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    z = lambda *s: torch.zeros(s, device="cuda")
    w, k, v, o, u = z(B, T, C), z(B, T, C), z(B, T, C), z(B, T, C), z(C)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    base = [B, T, C, P(w), P(u), P(k), P(v), None, P(o), None]
    assert lib.wkv_forward_dd(*base, 0, 0, s) == 0
    assert lib.wkv_forward_dd(*base, 0, 3, s) == 7       # no look-back kernel: WKV_ERR_ARG
    assert lib.wkv_forward_dd(*base, 2, 0, s) == 7       # io out of range
    bad = list(base)
    bad[3] = None
    assert lib.wkv_forward_dd(*bad, 0, 0, s) == 1        # rates missing
    bad = list(base)
    bad[8] = P(w)
    assert lib.wkv_forward_dd(*bad, 0, 0, s) == 4        # out on top of the rates
    st = z(3, B, C)
    ks = z(B, C)
    assert lib.wkv_step_dd(B, C, P(ks), P(u), P(ks), P(ks), P(st), P(z(B, C)), 0, s) == 0
    assert lib.wkv_step_dd(B, C, None, P(u), P(ks), P(ks), P(st), P(z(B, C)), 0, s) == 1
    assert lib.wkv_step_dd(B, C, P(ks), P(u), P(ks), P(ks), P(st), P(ks), 0, s) == 4
    torch.cuda.synchronize()


def test_dd_layer_shape_sampled():
    """The 8-layer model's layer shape (B=8, T=1024, C=768, fp32) through the
    automatic choice; every batch row on 24 sampled channels against the
    oracle (lanes are independent, so a column subset is exact)."""
    wl = I.WORKLOADS[1]
    say(f"dd layer shape B={wl.B} T={wl.T} C={wl.C}")
    w, u = I.params(wl, 0)
    k, v = I.kv(wl, 0)
    wt = I.decay_rates(wl, 0)
    got, gst = gpu_dd(wt, u, k, v, "f32")
    cols = np.random.default_rng(5).choice(wl.C, 24, replace=False)
    ref, rst = wkv_dd_recurrent(wt[:, :, cols], u[cols], k[:, :, cols], v[:, :, cols])
    assert_out_close(got[:, :, cols], ref, v[:, :, cols], F32_TOL)
    assert_state_close(gst[:, :, cols], rst, F32_TOL)

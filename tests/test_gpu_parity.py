"""Parity of the HIP path (through the C interface) with the float64 oracle,
element by element, on seeded inputs small enough for the oracle: ragged
sizes around every tile edge of both prefill kernels, initial states,
in-place states, split/resume, decode, bf16 I/O and extreme keys."""

import warnings

import numpy as np
import pytest
import torch

from oracle import sigmoid
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
# segments (32 tokens for T <= 512, 256 beyond; anchors every 8 segments), and C
# around both kernels' 32-channel groups (64 for bf16, and for the look-back's
# fp32 layout past 2048 tokens); every kernel runs every shape.
SHAPES = [
    (1, 1, 1), (2, 2, 7), (1, 3, 16), (3, 31, 33), (2, 32, 5), (2, 63, 48), (2, 64, 64),
    (2, 65, 17), (1, 255, 16), (1, 256, 32), (1, 257, 80), (2, 511, 24), (1, 1000, 40),
    (1, 2048, 31), (1, 2049, 96), (2, 3000, 100), (1, 4097, 16), (1, 513, 40), (2, 1152, 33),
    (1, 1153, 64), (2, 2304, 33), (1, 2400, 40),
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
                                   (3, 700, 32), (1, 2049, 66), (1, 130, 7), (1, 2500, 130),
                                   (1, 1, 512), (2, 9, 512), (1, 300, 1536), (2, 1029, 1024),
                                   (64, 300, 256)])
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


@pytest.mark.parametrize("gated", [False, True], ids=["plain", "gated"])
def test_bf16_tile_walk_from_state(gated):
    """The bf16 sequential scan's LDS-staged tile walk (C a multiple of 512,
    16-byte aligned rows): an initial state, a ragged last tile (T = 333 is
    41 tiles of 8 and 5 tokens), two 1 KiB row pieces per batch row, with and
    without the receptance gate."""
    B, T, C = 2, 333, 1024
    say(f"bf16 tile walk gated={gated}")
    w, u, k, v = make_case(WL4, B, T, C)
    k, v = I.round_to_bf16(k), I.round_to_bf16(v)
    s0 = random_state(B, C, 4)
    ds = dev_f32(s0)
    if gated:
        r = I.round_to_bf16(np.random.default_rng([62, T]).normal(0, 2, (B, T, C)).astype(np.float32))
        out, st = W.wkv_forward_gated(dev_f32(w), dev_f32(u), dev_io(k, "bf16"), dev_io(v, "bf16"),
                                      dev_io(r, "bf16"), state_in=ds, path="seq")
        ref, rst = wkv_recurrent(w, u, k, v, s0.astype(np.float64))
        ref = ref * sigmoid(r)
    else:
        out, st = W.wkv_forward_ex(dev_f32(w), dev_f32(u), dev_io(k, "bf16"), dev_io(v, "bf16"),
                                   ds, path="seq")
        ref, rst = wkv_recurrent(w, u, k, v, s0.astype(np.float64))
    torch.cuda.synchronize()
    assert_out_close(host64(out), ref, v, BF16_TOL)
    assert_state_close(host64(st), rst, F32_TOL * 10)


@pytest.mark.parametrize("B,T,C", [(1, 257, 32), (3, 512, 33), (2, 768, 96), (1, 769, 64),
                                   (2, 1023, 40), (1, 1024, 768), (2, 300, 7)])
@pytest.mark.parametrize("with_state", [False, True], ids=["empty", "state"])
def test_chunk_two_walkers(B, T, C, with_state):
    """fp32 chunked scan over two to four 256-token tiles, where a workgroup
    runs two walkers (the first half of the tiles from the initial state, the
    second half from the first walker's final state): odd tile counts, a
    ragged last tile, idle channel threads, several groups per row."""
    say(f"chunk two walkers B={B} T={T} C={C} state={with_state}")
    w, u, k, v = make_case(WL3, B, T, C)
    s0 = random_state(B, C, 6) if with_state else None
    got, gst = gpu_forward(w, u, k, v, "f32", state_in=s0, path="chunk")
    ref, rst = wkv_recurrent(w, u, k, v, None if s0 is None else s0.astype(np.float64))
    assert_out_close(got, ref, v, F32_TOL)
    assert_state_close(gst, rst, F32_TOL)


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


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("kmag", [60.0, 88.0, 1e4])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_extreme_keys(path, kmag, io):
    """No NaN/Inf and oracle agreement with keys far outside N(0, 1), at the
    workload tolerance at every magnitude, |k| = 1e4 included. Every kernel
    forms its exponent differences from key differences plus whole numbers
    times w, and the time-parallel paths keep their sub-chunk sums exact
    relative to each stored (rounded) maximum, so keys on the coarse grid of
    ulp(1e4) ~ 1e-3 cost no accuracy beyond the data's own (measured on MI355X:
    2.7e-7 on every fp32 path at |k| = 1e4)."""
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
    tol = tol_for(io)
    e = assert_out_close(got, ref, v, tol)
    say(f"  max normalised output error {e:.3e} (bound {tol:.1e})")
    assert np.isfinite(gst).all()
    assert_state_close(gst, rst, F32_TOL)


def test_auto_path_choice():
    """Large B*C goes to the sequential scan (the chunked scan for fp32 rows
    whose byte size is not a power of two, 512 <= T <= 2048); small B*C to the
    chunked scan up to T = 2048 and to the look-back scan beyond (the chunked
    scan when no workspace is given)."""
    # fp32 rows of 1.5 MiB: the chunked scan; rows of a power-of-two size: the walk
    assert W.wkv_select_path(256, 512, 768) == "chunk"
    assert W.wkv_select_path(256, 512, 1024) == "seq"
    assert W.wkv_select_path(512, 256, 768) == "seq"
    assert W.wkv_select_path(256, 512, 768, W.WKV_IO_BF16) == "seq"
    assert W.wkv_select_path(64, 4096, 4096, W.WKV_IO_BF16) == "seq"
    assert W.wkv_select_path(8, 1024, 768) == "chunk"
    assert W.wkv_select_path(4, 16384, 2048) == "lookback"
    assert W.wkv_select_path(1, 64, 768) == "chunk"
    assert W.wkv_select_path(4, 8, 64) == "seq"


def test_auto_takes_lookback_for_mid_length_fp32_with_more_groups_than_cus():
    """With a workspace, fp32 past 512 tokens (gated: from 1280) and up to
    2048 takes the look-back scan where the chunked scan's 32-channel groups
    outnumber the CUs by up to four to one: the choice itself at its edges,
    and the AUTO result (bit for bit that of the explicit look-back call, and
    against the oracle) on a plain and a gated shape just past one group per
    CU."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    b2 = 2 * cus // 32  # B with 2 * cus groups of C = 1024
    assert W.wkv_select_path(b2, 1024, 1024) == "lookback"
    assert W.wkv_select_path(b2, 513, 1024) == "lookback"
    assert W.wkv_select_path(b2, 512, 1024) == "chunk"
    assert W.wkv_select_path(b2, 2048, 1024) == "lookback"
    assert W.wkv_select_path(b2, 1024, 1024, W.WKV_IO_BF16) == "chunk"
    assert W.wkv_select_path(cus // 32, 1024, 1024) == "chunk"  # one group per CU
    assert W.wkv_select_path(4 * cus // 32, 1024, 1024) == "lookback"
    assert W.wkv_select_path(4 * cus // 32 + 1, 1024, 1024) == "chunk"

    B = cus // 24 + 1  # just past one group per CU at C = 768
    for gated, T in ((False, 640), (True, 1280)):
        say(f"auto look-back: B={B} T={T} C=768 gated={gated}")
        w, u, k, v = make_case(WL3, B, T, 768)
        ws = W.new_workspace(W.wkv_workspace_size(B, T, 768, W.WKV_IO_F32, "auto"), "cuda")
        assert ws.numel() >= W.wkv_workspace_size(B, T, 768, W.WKV_IO_F32, "lookback") > 0
        ref, rst = wkv_recurrent(w, u, k, v)
        args = [dev_f32(w), dev_f32(u), dev_f32(k), dev_f32(v)]
        if gated:
            r = np.random.default_rng([63, T]).normal(0, 2, (B, T, 768)).astype(np.float32)
            args.append(dev_f32(r))
            ref = ref * sigmoid(r)
            call = lambda path: W.wkv_forward_gated(*args, path=path, workspace=ws)
        else:
            call = lambda path: W.wkv_forward_ws(*args, path=path, workspace=ws)
        auto_out, auto_st = call("auto")
        lb_out, lb_st = call("lookback")
        torch.cuda.synchronize()
        assert W.wkv_workspace_status(ws) == 0
        assert torch.equal(auto_out, lb_out) and torch.equal(auto_st, lb_st)
        assert_out_close(host64(auto_out), ref, v, F32_TOL)
        assert_state_close(host64(auto_st), rst, F32_TOL)


def test_one_shot_calls_under_graph_capture_take_no_cached_workspace():
    """A one-shot AUTO call captured in a HIP graph takes no workspace from
    the binding's cache (checking it afterwards would synchronise the
    capturing stream), so AUTO picks a kernel that needs none: the replays
    give exactly the chunked scan's eager result, at a mid length where AUTO
    with a workspace takes the look-back scan and past 2048 tokens. An
    explicit look-back call without a workspace is refused during capture."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for B, T, C in ((cus // 24 + 1, 640, 768), (2, 2300, 96)):
        say(f"one-shot call under capture: B={B} T={T} C={C}")
        w, u, k, v = make_case(WL3, B, T, C)
        args = [dev_f32(w), dev_f32(u), dev_f32(k), dev_f32(v)]
        ref_out, ref_st = W.wkv_forward_ex(*args, path="chunk")
        out = torch.empty_like(ref_out)
        st = torch.empty_like(ref_st)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            W.wkv_forward_ex(*args, out=out, state_out=st)
        for rep in range(3):
            out.zero_()
            st.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, ref_out) and torch.equal(st, ref_st), f"replay {rep}"
    g2 = torch.cuda.CUDAGraph()
    with warnings.catch_warnings():
        warnings.simplefilter("ignore", UserWarning)  # the refused call leaves the graph empty
        with pytest.raises(ValueError, match="graph capture"):
            with torch.cuda.graph(g2):
                W.wkv_forward_ex(*args, out=out, state_out=st, path="lookback")


def _lookback_words(ws, groups):
    """The look-back workspace's control words (error, test word, the 64-bit
    layout claim) and every channel group's 64-bit ticket counter."""
    head = ws[:16].view(torch.int32).cpu().numpy().astype(np.int64) & 0xffffffff
    claim = int(ws[8:16].view(torch.int64).cpu().numpy()[0])
    tickets = ws[16:16 + 16 * groups].view(torch.int64).cpu().numpy().reshape(groups, 2)[:, 0]
    return head, claim, tickets


def test_lookback_workspace_claim_tickets_and_error_word():
    """The look-back workspace after n launches: it is claimed for its layout
    (G << 32 | S), every channel group's ticket counter has advanced by
    exactly S (segments per group) per launch, which is what gives each
    launch its own epoch, and the error word stays zero. T = 3000 takes the
    plain fp32 layout for sequences past 2048 tokens: 64-channel groups and
    256-token segments, so G = 2 * 2 and S = 12."""
    wl = WL3.scaled(B=2, T=3000, C=96)
    w, u = I.params(wl)
    k, v = I.kv(wl)
    ws = W.new_workspace(W.wkv_workspace_size(2, 3000, 96, W.WKV_IO_F32, "lookback"), "cuda")
    say("look-back workspace counters")
    ref, _ = wkv_recurrent(w, u, k, v)
    groups, S = 2 * ((96 + 63) // 64), (3000 + 255) // 256
    for n in range(3):
        out, _ = W.wkv_forward_ws(dev_f32(w), dev_f32(u), dev_f32(k), dev_f32(v), path="lookback",
                                  workspace=ws)
        torch.cuda.synchronize()
        assert_out_close(host64(out), ref, v, F32_TOL)
        head, claim, tickets = _lookback_words(ws, groups)
        assert head[0] == 0, "a look-back launch failed to chain its segments"
        assert claim == (groups << 32) | S
        assert np.all(tickets == (n + 1) * S), tickets
        assert W.wkv_workspace_status(ws) == 0


def test_lookback_workspace_of_another_layout_is_reported():
    """A workspace claimed by one look-back layout and then given sizes with
    another one, without being zero-filled again: the launch finishes, every
    output it could not chain is NaN (none is a plausible wrong value) and
    wkv_workspace_status reports WKV_ERR_LOOKBACK. Zero-filled again, the
    workspace serves the new sizes correctly."""
    a, b = (2, 3000, 96), (1, 4097, 40)
    nbytes = max(W.wkv_workspace_size(*x, W.WKV_IO_F32, "lookback") for x in (a, b))
    ws = W.new_workspace(nbytes, "cuda")
    for i, (B, T, C) in enumerate((a, b)):
        say(f"look-back layout claim {i}: B={B} T={T} C={C}")
        w, u, k, v = make_case(WL3, B, T, C, layer=i)
        ref, _ = wkv_recurrent(w, u, k, v)
        out, _ = W.wkv_forward_ws(dev_f32(w), dev_f32(u), dev_f32(k), dev_f32(v), path="lookback",
                                  workspace=ws)
        torch.cuda.synchronize()
        got = host64(out)
        if i == 0:
            assert_out_close(got, ref, v, F32_TOL)
            assert W.wkv_workspace_status(ws) == 0
        else:
            assert W.wkv_workspace_status(ws, clear=True) == W.WKV_ERR_LOOKBACK
            assert np.isnan(got[:, 256:]).all()
            ws.zero_()
            out, _ = W.wkv_forward_ws(dev_f32(w), dev_f32(u), dev_f32(k), dev_f32(v),
                                      path="lookback", workspace=ws)
            torch.cuda.synchronize()
            assert_out_close(host64(out), ref, v, F32_TOL)
            assert W.wkv_workspace_status(ws) == 0


def test_lookback_gated_and_plain_layouts_on_one_workspace():
    """Past 2048 tokens the gated and the plain forward chain their segments
    in different look-back layouts (32-channel pairs of four waves against
    64-channel rows of eight), so one workspace serves one of them at a time:
    the gated call after a plain one on the same, uncleared workspace is
    reported and its chained outputs are NaN; zero-filled again, it is right."""
    B, T, C = 2, 3000, 96
    w, u, k, v = make_case(WL3, B, T, C)
    r = np.random.default_rng([62, B, T, C]).normal(0, 2.0, (B, T, C)).astype(np.float32)
    ref, _ = wkv_recurrent(w, u, k, v)
    gref = ref * sigmoid(r.astype(np.float64))
    ws = W.new_workspace(W.wkv_workspace_size(B, T, C, W.WKV_IO_F32, "lookback"), "cuda")
    say("look-back plain then gated on one workspace")
    out, _ = W.wkv_forward_ws(dev_f32(w), dev_f32(u), dev_f32(k), dev_f32(v), path="lookback",
                              workspace=ws)
    torch.cuda.synchronize()
    assert_out_close(host64(out), ref, v, F32_TOL)
    assert W.wkv_workspace_status(ws) == 0
    out, _ = W.wkv_forward_gated(dev_f32(w), dev_f32(u), dev_f32(k), dev_f32(v), dev_f32(r),
                                 path="lookback", workspace=ws)
    torch.cuda.synchronize()
    assert W.wkv_workspace_status(ws, clear=True) == W.WKV_ERR_LOOKBACK
    assert np.isnan(host64(out)[:, 256:]).all()
    ws.zero_()
    out, _ = W.wkv_forward_gated(dev_f32(w), dev_f32(u), dev_f32(k), dev_f32(v), dev_f32(r),
                                 path="lookback", workspace=ws)
    torch.cuda.synchronize()
    assert_out_close(host64(out), gref, v, F32_TOL)
    assert W.wkv_workspace_status(ws) == 0


def test_lookback_wait_that_runs_out_is_reported_and_poisons_outputs():
    """Forced from the host through the workspace's test words: with nothing
    published and a bound of 64 polls, every wait for an earlier segment runs
    out. The launch still finishes, wkv_workspace_status reports
    WKV_ERR_LOOKBACK, the first segment's outputs are right and every later
    one is NaN (never a plausible value); with the test words cleared the same
    workspace works again."""
    B, T, C = 2, 3000, 96
    w, u, k, v = make_case(WL3, B, T, C)
    ref, _ = wkv_recurrent(w, u, k, v)
    ws = W.new_workspace(W.wkv_workspace_size(B, T, C, W.WKV_IO_F32, "lookback"), "cuda")
    ctl = ws[:16].view(torch.int32)
    ctl[1] = 1 | (64 << 8)   # publish nothing; 64 polls before a wait gives up
    say("look-back forced wait time-out")
    out, _ = W.wkv_forward_ws(dev_f32(w), dev_f32(u), dev_f32(k), dev_f32(v), path="lookback",
                              workspace=ws)
    torch.cuda.synchronize()
    got = host64(out)
    assert W.wkv_workspace_status(ws) == W.WKV_ERR_LOOKBACK
    assert W.wkv_workspace_status(ws, clear=True) == W.WKV_ERR_LOOKBACK
    assert W.wkv_workspace_status(ws) == 0
    assert_out_close(got[:, :256], ref[:, :256], v[:, :256], F32_TOL)
    assert np.isnan(got[:, 256:]).all()
    with pytest.raises(W.WKVError):
        W.check_workspace(_poisoned_again(ws, w, u, k, v))
    ctl[1] = 0
    W.wkv_workspace_status(ws, clear=True)
    out, _ = W.wkv_forward_ws(dev_f32(w), dev_f32(u), dev_f32(k), dev_f32(v), path="lookback",
                              workspace=ws)
    torch.cuda.synchronize()
    assert_out_close(host64(out), ref, v, F32_TOL)
    assert W.wkv_workspace_status(ws) == 0


def _poisoned_again(ws, w, u, k, v):
    """One more launch with the test words still set; returns the workspace."""
    W.wkv_forward_ws(dev_f32(w), dev_f32(u), dev_f32(k), dev_f32(v), path="lookback", workspace=ws)
    return ws


def test_lookback_calls_in_hip_graph_replay_exactly():
    """Look-back launches captured once in a HIP graph: every replay takes
    fresh tickets and epochs from the never-reset counters, so outputs and
    states are bit-identical to the eager calls' on every replay (fp32 past
    2048 tokens: the 64-channel-row layout), with eager work in between, and
    the workspaces report no error."""
    say("look-back graph capture")
    wl = WL3.scaled(B=2, T=2300, C=160)
    layers = []
    for layer in range(2):
        w, u = I.params(wl, layer)
        k, v = I.kv(wl, layer)
        layers.append((dev_f32(w), dev_f32(u), dev_f32(k), dev_f32(v)))
    calls = [W.ForwardCall(*L, path="lookback") for L in layers]
    for c in calls:
        c()
    torch.cuda.synchronize()
    eager = [(c.out.clone(), c.state_out.clone()) for c in calls]
    w, u = I.params(wl, 0)
    k, v = I.kv(wl, 0)
    ref, rst = wkv_recurrent(w, u, k, v)
    assert_out_close(host64(eager[0][0]), ref, v, F32_TOL)
    assert_state_close(host64(eager[0][1]), rst, F32_TOL)
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
        for c, (o, st) in zip(calls, eager):
            assert torch.equal(c.out.view(torch.int32), o.view(torch.int32)), f"replay {rep}"
            assert torch.equal(c.state_out.view(torch.int32), st.view(torch.int32)), f"replay {rep}"
        _ = W.wkv_forward(*layers[0])
    for c in calls:
        assert W.wkv_workspace_status(c.workspace) == 0


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

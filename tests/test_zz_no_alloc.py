"""wkv_forward_noalloc (for callers that cannot allocate): the look-back
workspace lives in the library's static device array. Called through the C
interface with ctypes, it must give exactly the outputs and final states of
wkv_forward_ws with a caller-owned workspace (same kernels), and meet the
oracle's tolerance, on calls in a row with shrinking sizes."""

import ctypes

import numpy as np
import pytest
import torch

from wkvtest import (F32_TOL, I, W, assert_out_close, assert_state_close, dev_f32, host64,
                     make_case, say, wkv_recurrent)

pytestmark = pytest.mark.gpu

P = ctypes.c_void_p
WL3 = I.WORKLOADS[3]


def _p(t):
    return None if t is None else P(t.data_ptr())


def _stream():
    return P(torch.cuda.current_stream().cuda_stream)


def _both(lib, B, T, C, path, layer):
    w, u, k, v = make_case(WL3, B, T, C, layer=layer)
    dw, du, dk, dv = dev_f32(w), dev_f32(u), dev_f32(k), dev_f32(v)
    out_a = torch.full((B, T, C), float("nan"), device="cuda")
    st_a = torch.full((3, B, C), float("nan"), device="cuda")
    out_b, st_b = torch.full_like(out_a, float("nan")), torch.full_like(st_a, float("nan"))
    nbytes = W.wkv_workspace_size(B, T, C, W.WKV_IO_F32, "lookback")
    ws = W.new_workspace(nbytes, "cuda")
    assert lib.wkv_forward_ws(B, T, C, _p(dw), _p(du), _p(dk), _p(dv), None, _p(out_a), _p(st_a),
                              W.WKV_IO_F32, path, _p(ws), nbytes, _stream()) == 0
    assert lib.wkv_forward_noalloc(B, T, C, _p(dw), _p(du), _p(dk), _p(dv), None, _p(out_b),
                                   _p(st_b), W.WKV_IO_F32, path, _stream()) == 0
    torch.cuda.synchronize()
    return (w, u, k, v), (out_a, st_a), (out_b, st_b)


@pytest.mark.parametrize("path", [W.WKV_PATH_LOOKBACK, W.WKV_PATH_AUTO], ids=["lookback", "auto"])
def test_noalloc_matches_workspace_call_on_shrinking_sizes(path):
    lib = W.load_library()
    for i, (B, T, C) in enumerate([(2, 4100, 96), (1, 2305, 40)]):
        say(f"noalloc call {i}: B={B} T={T} C={C} path={path}")
        (w, u, k, v), (oa, sa), (ob, sb) = _both(lib, B, T, C, path, layer=i)
        assert torch.equal(oa, ob), "outputs differ from wkv_forward_ws"
        assert torch.equal(sa, sb), "final states differ from wkv_forward_ws"
        ref, rst = wkv_recurrent(w, u, k, v)
        assert_out_close(host64(ob), ref, v, F32_TOL)
        assert_state_close(host64(sb), rst, F32_TOL)


def test_noalloc_rejects_lookback_beyond_its_array():
    """The long-context workload's batch widened 8 times needs a 235 MB look-back
    workspace: past the 32 MiB array, an explicit LOOKBACK is refused."""
    lib = W.load_library()
    say("noalloc oversize")
    B, T, C = 32, 16384, 2048
    assert W.wkv_workspace_size(B, T, C, W.WKV_IO_F32, "lookback") > 32 << 20
    t = torch.zeros(4, device="cuda")
    assert lib.wkv_forward_noalloc(B, T, C, _p(t), _p(t), _p(t), _p(t), None, _p(t), None,
                                   W.WKV_IO_F32, W.WKV_PATH_LOOKBACK, _stream()) == 8


def test_noalloc_auto_mid_length_lookback_between_other_layouts():
    """Where AUTO takes the look-back scan below 2049 tokens (fp32 with more
    32-channel groups than CUs, at most four per CU), the static array serves
    it too: a call of that kind between two calls of other look-back layouts
    (each call clears the part of the array it uses) matches wkv_forward_ws
    bit for bit and the oracle."""
    lib = W.load_library()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    mid = (cus // 24 + 1, 640, 768)  # just past one 32-channel group per CU
    assert W.wkv_select_path(*mid) == "lookback"
    for i, (B, T, C) in enumerate([(1, 2305, 40), mid, (2, 4100, 96)]):
        say(f"noalloc auto call {i}: B={B} T={T} C={C}")
        (w, u, k, v), (oa, sa), (ob, sb) = _both(lib, B, T, C, W.WKV_PATH_AUTO, layer=i)
        assert torch.equal(oa, ob), "outputs differ from wkv_forward_ws"
        assert torch.equal(sa, sb), "final states differ from wkv_forward_ws"
        ref, rst = wkv_recurrent(w, u, k, v)
        assert_out_close(host64(ob), ref, v, F32_TOL)
        assert_state_close(host64(sb), rst, F32_TOL)

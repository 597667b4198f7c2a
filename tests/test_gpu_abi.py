"""The C interface's conventions, exercised through ctypes with real device
pointers: status codes for bad arguments, zero sizes, T = 0, NULL states."""

import ctypes

import numpy as np
import pytest
import torch

from wkvtest import F32_TOL, I, W, assert_out_close, dev_f32, host64, make_case, say, wkv_recurrent

pytestmark = pytest.mark.gpu

P = ctypes.c_void_p


def ptr(t, offset_bytes=0):
    return None if t is None else P(t.data_ptr() + offset_bytes)


def stream():
    return P(torch.cuda.current_stream().cuda_stream)


@pytest.fixture(scope="module")
def lib():
    return W.load_library()


@pytest.fixture()
def case():
    B, T, C = 2, 40, 24
    w, u, k, v = make_case(I.WORKLOADS[0], B, T, C)
    d = dict(B=B, T=T, C=C, w=dev_f32(w), u=dev_f32(u), k=dev_f32(k), v=dev_f32(v),
             out=torch.empty((B, T, C), device="cuda"), st=torch.empty((3, B, C), device="cuda"))
    d["host"] = (w, u, k, v)
    return d


def call_fwd(lib, c, **over):
    a = dict(B=c["B"], T=c["T"], C=c["C"], w=ptr(c["w"]), u=ptr(c["u"]), k=ptr(c["k"]),
             v=ptr(c["v"]), s_in=None, out=ptr(c["out"]), s_out=ptr(c["st"]))
    a.update(over)
    return lib.wkv_forward(a["B"], a["T"], a["C"], a["w"], a["u"], a["k"], a["v"], a["s_in"],
                           a["out"], a["s_out"], stream())


def test_valid_call_ok(lib, case):
    say("abi: valid call")
    assert call_fwd(lib, case) == 0
    torch.cuda.synchronize()
    w, u, k, v = case["host"]
    ref, _ = wkv_recurrent(w, u, k, v)
    assert_out_close(host64(case["out"]), ref, v, F32_TOL)


def test_error_codes(lib, case):
    say("abi: error codes")
    assert call_fwd(lib, case, w=None) == 1
    assert call_fwd(lib, case, k=None) == 1
    assert call_fwd(lib, case, out=None) == 1
    assert call_fwd(lib, case, B=-1) == 2
    assert call_fwd(lib, case, T=1 << 62) == 2
    assert call_fwd(lib, case, k=ptr(case["k"], 2)) == 3       # not 4-byte aligned
    assert call_fwd(lib, case, out=ptr(case["k"])) == 4        # out on top of k
    assert call_fwd(lib, case, out=ptr(case["v"], 4)) == 4     # partial overlap
    assert call_fwd(lib, case, s_out=ptr(case["w"])) == 4      # state_out on an input
    s_in = torch.zeros((3, case["B"], case["C"]), device="cuda")
    assert call_fwd(lib, case, s_in=ptr(s_in), s_out=ptr(s_in, 4)) == 4  # shifted overlap
    rc = lib.wkv_forward_ex(1, 1, 1, ptr(case["w"]), ptr(case["u"]), ptr(case["k"]),
                            ptr(case["v"]), None, ptr(case["out"]), None, 9, 0, stream())
    assert rc == 7
    for code in range(8):
        assert W.wkv_status_string(code)
    torch.cuda.synchronize()


def test_zero_sizes_are_noops(lib, case):
    say("abi: zero sizes")
    case["out"].fill_(7.0)
    assert call_fwd(lib, case, B=0) == 0
    assert call_fwd(lib, case, C=0) == 0
    assert lib.wkv_step(0, 5, None, None, None, None, None, None, stream()) == 0
    torch.cuda.synchronize()
    assert torch.all(case["out"] == 7.0)


def test_t0_copies_or_empties_state(lib, case):
    say("abi: T=0")
    s_in = dev_f32(np.random.default_rng(3).normal(size=(3, case["B"], case["C"])))
    assert call_fwd(lib, case, T=0, s_in=ptr(s_in), k=None, v=None, out=None) == 0
    torch.cuda.synchronize()
    assert torch.equal(case["st"], s_in)
    assert call_fwd(lib, case, T=0, k=None, v=None, out=None) == 0
    torch.cuda.synchronize()
    st = host64(case["st"])
    assert np.all(st[0] == 0) and np.all(st[1] == 0) and np.all(st[2] <= -1e37)


def test_null_state_out_and_empty_state_in(lib, case):
    say("abi: NULL state_out")
    assert call_fwd(lib, case, s_out=None) == 0
    empty = dev_f32(np.stack([np.zeros((case["B"], case["C"]))] * 2
                             + [np.full((case["B"], case["C"]), -1e38)]))
    out2 = torch.empty_like(case["out"])
    assert call_fwd(lib, case, s_in=ptr(empty), out=ptr(out2)) == 0
    torch.cuda.synchronize()
    assert torch.equal(case["out"], out2)


def test_step_error_codes(lib, case):
    say("abi: step error codes")
    B, C = case["B"], case["C"]
    k = case["k"][:, 0].contiguous()
    v = case["v"][:, 0].contiguous()
    st = torch.zeros((3, B, C), device="cuda")
    out = torch.empty((B, C), device="cuda")
    args = [ptr(case["w"]), ptr(case["u"]), ptr(k), ptr(v), ptr(st), ptr(out)]
    assert lib.wkv_step(B, C, *args, stream()) == 0
    bad = list(args)
    bad[5] = ptr(st)
    assert lib.wkv_step(B, C, *bad, stream()) == 4
    bad = list(args)
    bad[4] = None
    assert lib.wkv_step(B, C, *bad, stream()) == 1
    torch.cuda.synchronize()


def test_binding_rejects_bad_tensors():
    say("binding checks")
    w = torch.ones(8, device="cuda")
    k = torch.zeros((1, 4, 8), device="cuda")
    with pytest.raises(TypeError):
        W.wkv_forward(w, w, k.double(), k.double())
    with pytest.raises(ValueError):
        W.wkv_forward(w, w, k, k.transpose(1, 2).contiguous().transpose(1, 2))
    with pytest.raises(ValueError):
        W.wkv_forward(torch.ones(7, device="cuda"), w, k, k)


def test_forward_ws_workspace_rules(lib, case):
    say("abi: workspace")
    B, T, C = case["B"], case["T"], case["C"]
    need = lib.wkv_workspace_size(B, T, C, 0, W.WKV_PATH_LOOKBACK)
    assert need > 256
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    base = [B, T, C, ptr(case["w"]), ptr(case["u"]), ptr(case["k"]), ptr(case["v"]), None,
            ptr(case["out"]), ptr(case["st"]), 0, W.WKV_PATH_LOOKBACK]
    assert lib.wkv_forward_ws(*base, ptr(ws), need, stream()) == 0
    torch.cuda.synchronize()
    w, u, k, v = case["host"]
    ref, _ = wkv_recurrent(w, u, k, v)
    assert_out_close(host64(case["out"]), ref, v, F32_TOL)
    assert lib.wkv_forward_ws(*base, ptr(ws), need - 8, stream()) == 8     # too small
    assert lib.wkv_forward_ws(*base, None, 0, stream()) == 8               # missing
    assert lib.wkv_forward_ex(*base, stream()) == 8                        # no workspace argument
    assert lib.wkv_forward_ws(*base, ptr(ws, 64), need - 64, stream()) == 3  # not 256-aligned
    assert lib.wkv_forward_ws(*base, ptr(case["out"]), need, stream()) == 4  # on top of out
    seq = list(base)
    seq[-1] = W.WKV_PATH_SEQ
    assert lib.wkv_forward_ws(*seq, None, 0, stream()) == 0              # seq needs none
    torch.cuda.synchronize()

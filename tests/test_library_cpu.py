"""Host-side checks that need no GPU: libwkv.so loads, exports every function
include/wkv.h declares, and its argument validation answers with the
documented status codes before touching the device. Also checks the seeded
input generators."""

import ctypes
import os
import re

import numpy as np
import pytest
import torch

import wkv_recurrence_scan_amd as W
from wkv_recurrence_scan_amd import inputs as I

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wkv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(wkv_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    lib = ctypes.CDLL(W.LIBRARY_PATH)
    names = declared_functions()
    assert len(names) >= 9, names
    for n in names:
        assert hasattr(lib, n), f"libwkv.so does not export {n}"


def test_header_compiles_as_c():
    import shutil
    import subprocess
    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("no C compiler")
    src = '#include "wkv.h"\nint main(void){return wkv_abi_version() == 1 ? 0 : 1;}\n'
    r = subprocess.run([cc, "-std=c99", "-fsyntax-only", "-D__HIP_PLATFORM_AMD__", "-I",
                        os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", "-x", "c", "-"],
                       input=src, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_validation_codes_without_device():
    lib = W.load_library()
    nul = None
    assert lib.wkv_abi_version() == 1
    assert lib.wkv_forward(-1, 1, 1, nul, nul, nul, nul, nul, nul, nul, nul) == 2
    assert lib.wkv_forward(1 << 40, 1 << 20, 1 << 10, nul, nul, nul, nul, nul, nul, nul, nul) == 2
    assert lib.wkv_forward(0, 5, 5, nul, nul, nul, nul, nul, nul, nul, nul) == 0
    assert lib.wkv_forward(2, 5, 0, nul, nul, nul, nul, nul, nul, nul, nul) == 0
    assert lib.wkv_forward(1, 2, 3, nul, nul, nul, nul, nul, nul, nul, nul) == 1
    assert lib.wkv_forward_ex(1, 1, 1, nul, nul, nul, nul, nul, nul, nul, 2, 0, nul) == 7
    assert lib.wkv_forward_ex(1, 1, 1, nul, nul, nul, nul, nul, nul, nul, 0, 4, nul) == 7
    assert lib.wkv_step(-2, 4, nul, nul, nul, nul, nul, nul, nul) == 2
    assert lib.wkv_step(2, 4, nul, nul, nul, nul, nul, nul, nul) == 1
    # fake, never-dereferenced addresses: alignment and overlap are decided on the host
    a = 0x10000000
    P = ctypes.c_void_p
    assert lib.wkv_forward(1, 4, 4, P(a), P(a + 64), P(a + 2 + 128), P(a + 256), nul,
                           P(a + 512), nul, nul) == 3
    assert lib.wkv_forward(1, 4, 4, P(a), P(a + 64), P(a + 128), P(a + 256), nul,
                           P(a + 128 + 32), nul, nul) == 4
    assert lib.wkv_select_path(1 << 30, 1 << 30, 1 << 10, 0) == -2
    assert lib.wkv_select_path(-1, 4, 4, 0) == -2
    assert lib.wkv_select_path(1, 4, 4, 9) == -7
    for code in range(9):
        assert lib.wkv_status_string(code)


def test_workspace_size_and_requirement_without_device():
    lib = W.load_library()
    P = ctypes.c_void_p
    seq, chunk, lookback = W.WKV_PATH_SEQ, W.WKV_PATH_CHUNK, W.WKV_PATH_LOOKBACK
    assert lib.wkv_workspace_size(8, 1024, 768, 0, seq) == 0
    assert lib.wkv_workspace_size(8, 1024, 768, 0, chunk) == 0
    n = lib.wkv_workspace_size(8, 1024, 768, 0, lookback)
    # control words (16 B + 16 B per 32-channel group, rounded up to 256 B) and
    # 7 tagged 8-byte words per (lane, segment): an aggregate (n, d, m) and an
    # inclusive prefix (n, d, base, age); T = 1024 uses 256-token segments
    groups = 8 * 768 // 32
    assert n == ((16 + 16 * groups + 255) // 256) * 256 + 8 * 768 * (1024 // 256) * 7 * 8
    # past 2048 tokens the plain fp32 form takes 64-channel groups and the
    # gated one 32-channel groups (256-token segments both): the size covers
    # the larger, here the 64-channel layout's 128 word columns per row of 96
    ctrl = lambda g: ((16 + 16 * g + 255) // 256) * 256  # noqa: E731
    S = (3000 + 255) // 256
    assert lib.wkv_workspace_size(2, 3000, 96, 0, lookback) == max(
        ctrl(2 * 3) + 2 * 96 * S * 7 * 8, ctrl(2 * 2) + 2 * 128 * S * 7 * 8)
    assert lib.wkv_workspace_size(8, 0, 768, 0, lookback) == 0
    assert lib.wkv_workspace_size(8, 1024, 768, 5, lookback) < 0
    assert lib.wkv_workspace_size(-1, 1024, 768, 0, lookback) < 0
    a = 0x10000000
    args = [P(a), P(a + 4096), P(a + 8192), P(a + 8192 + 65536), None, P(a + 8192 + 2 * 65536), None]
    # the look-back kernel without (enough) workspace is refused before any device call
    assert lib.wkv_forward_ex(1, 64, 256, *args, 0, lookback, None) == 8
    assert lib.wkv_forward_ws(1, 64, 256, *args, 0, lookback, P(a + (1 << 24)), 64, None) == 8
    assert lib.wkv_forward_ws(1, 64, 256, *args, 0, lookback, P((a + (1 << 24)) | 8), 1 << 20,
                              None) == 3
    assert lib.wkv_forward_ws(1, 64, 256, *args, 0, lookback, P(a + 8192), 1 << 20, None) == 4


def test_backward_workspace_and_validation_without_device():
    lib = W.load_library()
    P = ctypes.c_void_p
    # per-lane partial sums (rounded up to 256 B) + one 16-byte checkpoint per
    # (lane, chunk of 8 tokens)
    lanes = 256 * 768
    assert lib.wkv_backward_workspace_size(256, 512, 768) == \
        ((8 * lanes + 255) // 256) * 256 + (512 // 8) * lanes * 16
    assert lib.wkv_backward_workspace_size(2, 9, 4) == 256 + 2 * 8 * 16
    assert lib.wkv_backward_workspace_size(-1, 9, 4) < 0
    assert lib.wkv_backward_workspace_size(3, 9, 0) == 0
    nul = None
    a = 0x10000000
    args = [P(a), P(a + 4096)] + [P(a + (i + 2) * (1 << 20)) for i in range(2)]
    # B, T, C, w, u, k, v, r, state_in, state_out, gstate_out, gout, gk, gv, gr, gw, gu,
    # gstate_in
    base = [2, 9, 4, args[0], args[1], args[2], args[3], nul, nul, nul, nul,
            P(a + 5 * (1 << 20)), P(a + 6 * (1 << 20)), P(a + 7 * (1 << 20)), nul,
            P(a + 8 * (1 << 20)), P(a + 8 * (1 << 20) + 256), nul]
    assert lib.wkv_backward(-1, *base[1:], nul, 0, nul) == 2
    assert lib.wkv_backward(*base, nul, 0, nul) == 8                     # no workspace
    bad = list(base)
    bad[3] = nul
    assert lib.wkv_backward(*bad, nul, 0, nul) == 1                      # w missing
    bad = list(base)
    bad[10] = P(a + 9 * (1 << 20))                                       # gradient without state
    assert lib.wkv_backward(*bad, P(a + (1 << 28)), 1 << 20, nul) == 1
    bad = list(base)
    bad[7] = P(a + 10 * (1 << 20))                                       # r without dL/dr
    assert lib.wkv_backward(*bad, P(a + (1 << 28)), 1 << 20, nul) == 1
    bad = list(base)
    bad[13] = bad[5]                                                     # gv on top of k
    assert lib.wkv_backward(*bad, P(a + (1 << 28)), 1 << 20, nul) == 4
    assert lib.wkv_backward(*base, P(a + (1 << 28) + 8), 1 << 20, nul) == 3  # misaligned workspace


def test_gated_entry_points_validate_without_device():
    lib = W.load_library()
    P = ctypes.c_void_p
    nul = None
    a = 0x10000000
    w, u, k, v, r = P(a), P(a + 4096), P(a + 8192), P(a + 8192 + 4096), P(a + 8192 + 8192)
    out = P(a + 8192 + 3 * 4096)
    # B, T, C, w, u, k, v, r, state_in, out, state_out, io, path, workspace, bytes, stream
    assert lib.wkv_forward_gated(1, 4, 4, w, u, k, v, nul, nul, out, nul, 0, 1, nul, 0, nul) == 1
    assert lib.wkv_forward_gated(1, 4, 4, w, u, k, v, r, nul, r, nul, 0, 1, nul, 0, nul) == 4
    assert lib.wkv_forward_gated(1, 4, 4, w, u, k, v, P(a + 8192 + 8194), nul, out, nul, 0, 1,
                                 nul, 0, nul) == 3
    # B, C, w, u, k, v, r, state, out, io, stream
    assert lib.wkv_step_gated(2, 4, w, u, k, v, nul, P(a + 65536), out, 0, nul) == 1
    assert lib.wkv_step_gated(2, 4, w, u, k, v, r, P(a + 65536), out, 3, nul) == 7


def test_per_token_decay_entry_points_validate_without_device():
    lib = W.load_library()
    P = ctypes.c_void_p
    nul = None
    a = 0x10000000
    w, u, k, v = P(a), P(a + 4096), P(a + 8192), P(a + 12288)
    out = P(a + 16384)
    # B, T, C, w, u, k, v, state_in, out, state_out, io, path, stream
    assert lib.wkv_forward_dd(1, 4, 4, w, u, k, v, nul, out, nul, 0, 3, nul) == 7  # no look-back
    assert lib.wkv_forward_dd(1, 4, 4, w, u, k, v, nul, out, nul, 2, 0, nul) == 7
    assert lib.wkv_forward_dd(-1, 4, 4, w, u, k, v, nul, out, nul, 0, 0, nul) == 2
    assert lib.wkv_forward_dd(0, 4, 4, nul, nul, nul, nul, nul, nul, nul, 0, 0, nul) == 0
    assert lib.wkv_forward_dd(1, 4, 4, nul, u, k, v, nul, out, nul, 0, 0, nul) == 1
    assert lib.wkv_forward_dd(1, 4, 4, w, u, k, v, nul, w, nul, 0, 0, nul) == 4
    assert lib.wkv_forward_dd(1, 4, 4, P(a + 2), u, k, v, nul, out, nul, 0, 0, nul) == 3
    # B, C, w, u, k, v, state, out, io, stream
    assert lib.wkv_step_dd(2, 4, nul, u, k, v, P(a + 65536), out, 0, nul) == 1
    assert lib.wkv_step_dd(2, 4, w, u, k, v, P(a + 65536), w, 0, nul) == 4
    assert lib.wkv_step_dd(2, 4, w, u, k, v, P(a + 65536), out, 5, nul) == 7


def test_matrix_entry_points_validate_without_device():
    lib = W.load_library()
    P = ctypes.c_void_p
    nul = None
    a = 0x10000000
    w, k, v, r, out = P(a), P(a + 8192), P(a + 16384), P(a + 24576), P(a + 32768)
    # B, T, H, D, w, k, v, r, state_in, out, state_out, workspace, bytes, stream
    assert lib.wkv_matrix_forward(1, 2, 1, 32, w, k, v, r, nul, out, nul, nul, 0, nul) == 2
    assert lib.wkv_matrix_forward(-1, 2, 1, 64, w, k, v, r, nul, out, nul, nul, 0, nul) == 2
    assert lib.wkv_matrix_forward(0, 2, 1, 64, nul, nul, nul, nul, nul, nul, nul, nul, 0, nul) == 0
    assert lib.wkv_matrix_forward(1, 2, 1, 64, w, k, v, nul, nul, out, nul, nul, 0, nul) == 1
    assert lib.wkv_matrix_forward(1, 2, 1, 64, w, k, v, r, nul, k, nul, nul, 0, nul) == 4
    assert lib.wkv_matrix_forward(1, 2, 1, 64, P(a + 4), k, v, r, nul, out, nul, nul, 0, nul) == 3
    assert lib.wkv_matrix_workspace_size(1, 2, 1, 16) == -2
    # more heads than the 32-bit chunk offsets of the prefill kernels cover
    assert lib.wkv_matrix_forward(1, 1, (1 << 22) + 1, 64, w, k, v, r, nul, out, nul, nul, 0, nul) == 2
    assert lib.wkv_matrix_workspace_size(1, 1, (1 << 22) + 1, 64) == -2
    # B, H, D, w, k, v, r, state, out, stream
    assert lib.wkv_matrix_step(1, 1, 16, w, k, v, r, P(a + 65536), out, nul) == 2
    assert lib.wkv_matrix_step(1, 1, 64, w, k, v, r, nul, out, nul) == 1
    assert lib.wkv_matrix_step(1, 1, 64, w, k, v, r, P(a + 65536), w, nul) == 4


def test_token_shift_validates_without_device():
    lib = W.load_library()
    P = ctypes.c_void_p
    nul = None
    a = 0x10000000
    mu, x, xp, out, last = P(a), P(a + 4096), P(a + 8192), P(a + 16384), P(a + 65536)
    f32 = W.WKV_IO_F32
    # B, T, C, P, mu, x, x_prev, out, x_last, io, stream
    assert lib.wkv_token_shift(1, 2, 8, 0, mu, x, xp, out, last, f32, nul) == 2
    assert lib.wkv_token_shift(1, 2, 8, 9, mu, x, xp, out, last, f32, nul) == 2
    assert lib.wkv_token_shift(-1, 2, 8, 4, mu, x, xp, out, last, f32, nul) == 2
    assert lib.wkv_token_shift(1, 2, 8, 4, mu, x, xp, out, last, 5, nul) == 7
    assert lib.wkv_token_shift(0, 2, 8, 4, nul, nul, nul, nul, nul, f32, nul) == 0
    assert lib.wkv_token_shift(1, 2, 8, 4, mu, x, xp, nul, last, f32, nul) == 1
    assert lib.wkv_token_shift(1, 2, 8, 4, mu, P(a + 4098), xp, out, last, f32, nul) == 3
    # out over x; x_last inside x; x_last overlapping x_prev without being it
    assert lib.wkv_token_shift(1, 2, 8, 4, mu, x, xp, P(a + 4096 + 32), last, f32, nul) == 4
    assert lib.wkv_token_shift(1, 2, 8, 4, mu, x, xp, out, P(a + 4096 + 16), f32, nul) == 4
    assert lib.wkv_token_shift(1, 2, 8, 4, mu, x, xp, out, P(a + 8192 + 8), f32, nul) == 4


def test_checkpoint_entry_points_validate_without_device():
    lib = W.load_library()
    P = ctypes.c_void_p
    nul = None
    assert lib.wkv_ckpt_bytes(8, 1024, 768) == (1024 // 8) * 8 * 768 * 16
    assert lib.wkv_ckpt_bytes(2, 9, 3) == 2 * 2 * 3 * 16      # ceil(9 / 8) chunks
    assert lib.wkv_ckpt_bytes(-1, 8, 8) < 0
    a = 0x10000000
    w, u, k, v, out, ck = P(a), P(a + 4096), P(a + 8192), P(a + 16384), P(a + 24576), P(a + 65536)
    # B, T, C, w, u, k, v, r, state_in, out, state_out, ckpt, path, stream
    base = [1, 16, 64, w, u, k, v, nul, nul, out, nul]
    assert lib.wkv_forward_ckpt(*base, ck, W.WKV_PATH_LOOKBACK, nul) == 7
    assert lib.wkv_forward_ckpt(*base, nul, W.WKV_PATH_AUTO, nul) == 1
    assert lib.wkv_forward_ckpt(*base, P(a + 65536 + 8), W.WKV_PATH_AUTO, nul) == 3
    assert lib.wkv_forward_ckpt(*base, out, W.WKV_PATH_AUTO, nul) == 4
    # B, T, C, w, u, k, v, r, state_in, state_out, gstate_out, gout, ckpt, gk, gv, gr, gw, gu,
    # gstate_in, workspace, bytes, stream
    g, gk, gv, gw, gu = P(a + 32768), P(a + 40960), P(a + 49152), P(a + 57344), P(a + 61440)
    bwd = [1, 16, 64, w, u, k, v, nul, nul, nul, nul, g]
    rest = [gk, gv, nul, gw, gu, nul, P(a + (1 << 24)), 1 << 20, nul]
    assert lib.wkv_backward_ckpt(*bwd, nul, *rest) == 1
    assert lib.wkv_backward_ckpt(*bwd, P(a + 65536 + 4), *rest) == 3
    assert lib.wkv_backward_ckpt(*bwd, gk, *rest) == 4


def test_decay_backward_entry_points_validate_without_device():
    """wkv_backward_dd's host-side checks (they run before any device call):
    sizes, missing pointers, alignment, overlaps and the workspace."""
    lib = W.load_library()
    P = ctypes.c_void_p
    nul = None
    B, T, C = 2, 100, 16  # few lanes, T >= 64: the segmented plan needs a workspace
    need = lib.wkv_backward_dd_workspace_size(B, T, C)
    assert need > 0
    assert lib.wkv_backward_dd_workspace_size(-1, T, C) < 0
    assert lib.wkv_backward_dd_workspace_size(B, T, 0) == 0
    a = 0x10000000
    seq = B * T * C * 4
    w, k, v, g, gk, gv, gw = (P(a + i * seq) for i in range(7))
    u, gu = P(a + 7 * seq), P(a + 7 * seq + 256)
    ws = P(a + (1 << 24))
    # B, T, C, w, u, k, v, state_in, state_out, gstate_out, gout, gk, gv, gw, gu, gstate_in,
    # workspace, bytes, stream
    base = [B, T, C, w, u, k, v, nul, nul, nul, g, gk, gv, gw, gu, nul]
    bad = list(base)
    bad[3] = nul                                                         # w missing
    assert lib.wkv_backward_dd(*bad, ws, need, nul) == 1
    bad = list(base)
    bad[8] = P(a + (1 << 23))                                            # state_out without gradient
    assert lib.wkv_backward_dd(*bad, ws, need, nul) == 1
    bad = list(base)
    bad[13] = P(a + 3 * seq + 2)                                         # gw misaligned
    assert lib.wkv_backward_dd(*bad, ws, need, nul) == 3
    bad = list(base)
    bad[13] = k                                                          # gw on top of k
    assert lib.wkv_backward_dd(*bad, ws, need, nul) == 4
    assert lib.wkv_backward_dd(*base, ws, need - 8, nul) == 8            # workspace too small
    assert lib.wkv_backward_dd(*base, nul, 0, nul) == 8
    assert lib.wkv_backward_dd(*base, P(a + (1 << 24) + 8), need, nul) == 3  # not 256-aligned
    assert lib.wkv_backward_dd(-1, T, C, *base[3:], ws, need, nul) == 2


def test_decay_checkpoint_entry_points_validate_without_device():
    lib = W.load_library()
    P = ctypes.c_void_p
    nul = None
    a = 0x10000000
    B, T, C = 1, 16, 64
    seq = B * T * C * 4
    w, k, v, out = (P(a + i * seq) for i in range(4))
    u, ck = P(a + 4 * seq), P(a + 65536)
    # B, T, C, w, u, k, v, state_in, out, state_out, ckpt, path, stream
    base = [B, T, C, w, u, k, v, nul, out, nul]
    assert lib.wkv_forward_dd_ckpt(*base, ck, W.WKV_PATH_LOOKBACK, nul) == 7  # no look-back
    assert lib.wkv_forward_dd_ckpt(*base, nul, W.WKV_PATH_AUTO, nul) == 1     # ckpt missing
    assert lib.wkv_forward_dd_ckpt(*base, P(a + 65536 + 8), W.WKV_PATH_AUTO, nul) == 3
    assert lib.wkv_forward_dd_ckpt(*base, out, W.WKV_PATH_AUTO, nul) == 4     # ckpt on out
    # B, T, C, w, u, k, v, state_in, state_out, gstate_out, gout, ckpt, gk, gv, gw, gu,
    # gstate_in, workspace, bytes, stream
    g, gk, gv, gw = (P(a + (8 + i) * seq) for i in range(4))
    gu = P(a + 12 * seq)
    bwd = [B, T, C, w, u, k, v, nul, nul, nul, g]
    rest = [gk, gv, gw, gu, nul, P(a + (1 << 24)), 1 << 20, nul]
    assert lib.wkv_backward_dd_ckpt(*bwd, nul, *rest) == 1                   # ckpt missing
    assert lib.wkv_backward_dd_ckpt(*bwd, P(a + 65536 + 4), *rest) == 3      # misaligned
    assert lib.wkv_backward_dd_ckpt(*bwd, gk, *rest) == 4                    # an output on it


def test_per_token_decay_rates_are_seeded_and_positive():
    wl = I.WORKLOADS[1].scaled(B=3, T=50, C=32)
    r1 = I.decay_rates(wl)
    r2 = I.decay_rates(wl, rows=[1])
    assert np.array_equal(r1[1], r2[0]) and (r1 > 0).all()
    wc, _ = I.params(wl)
    ratio = np.log(r1 / wc[None, None, :])
    assert abs(ratio.std() - I.DD_LOG_STD) < 0.02 and abs(ratio.mean()) < 0.02
    rb = I.decay_rates(I.WORKLOADS[4].scaled(B=1, T=8, C=16))
    assert np.array_equal(I.round_to_bf16(rb), rb)
    assert I.decode_decay_rates(I.WORKLOADS[2].scaled(B=2, C=8), steps=5).shape == (5, 2, 8)


def test_inputs_are_seeded_and_row_independent():
    wl = I.WORKLOADS[3].scaled(B=3, T=20, C=16)
    k1, v1 = I.kv(wl)
    k2, v2 = I.kv(wl, rows=[2])
    assert np.array_equal(k1[2], k2[0]) and np.array_equal(v1[2], v2[0])
    w1, u1 = I.params(wl)
    w2, u2 = I.params(wl)
    assert np.array_equal(w1, w2) and np.array_equal(u1, u2)
    assert w1.min() >= 1e-3 * 0.999 and w1.max() <= 8.0 * 1.001
    k3, _ = I.kv(wl, layer=1)
    assert not np.array_equal(k3, k1)


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).normal(0, 30, 100000).astype(np.float32)
    x[:4] = [1.00390625, 1.01171875, -2.0078125, 3.0]  # exact ties and exact values
    ours = I.round_to_bf16(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(ours, theirs)
    bits = I.bf16_bits(ours)
    back = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(back, ours)


def test_stress_workload_distribution():
    wl = I.WORKLOADS[4].scaled(B=2, T=256, C=256)
    k, v = I.kv(wl)
    spikes = np.abs(k) == 60.0
    assert 0.007 < spikes.mean() < 0.013
    assert np.abs(k[~spikes]).max() <= 20.0
    assert np.array_equal(I.round_to_bf16(k), k)


def test_autograd_entry_rejects_host_tensors():
    """The autograd entry point validates like the prefill it wraps: host
    tensors are refused before any GPU call."""
    import torch

    import wkv_recurrence_scan_amd as W

    z = torch.zeros((1, 4, 8))
    with pytest.raises(ValueError, match="GPU"):
        W.wkv(torch.zeros(8), torch.zeros(8), z, z)

"""ctypes binding of libwkv.so (include/wkv.h): argument marshalling only.

Each function here has the name of the C entry point it calls and does no
arithmetic of the operator: it checks that the torch tensors it was given have
the device, dtype, shape and layout the C interface documents, allocates the
outputs the caller did not supply, and passes raw device pointers plus the
current HIP stream of the tensors' device. Everything else happens in the HIP
kernels behind the C interface. There is no fallback: if the library cannot be
loaded, every call raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY_PATH = os.path.join(_HERE, "libwkv.so")

WKV_IO_F32, WKV_IO_BF16 = 0, 1
WKV_PATH_AUTO, WKV_PATH_SEQ, WKV_PATH_CHUNK, WKV_PATH_LOOKBACK = 0, 1, 2, 3
_PATHS = {"auto": WKV_PATH_AUTO, "seq": WKV_PATH_SEQ, "chunk": WKV_PATH_CHUNK,
          "lookback": WKV_PATH_LOOKBACK}
_PATH_NAMES = {v: k for k, v in _PATHS.items()}

_lib = None


class WKVError(RuntimeError):
    """A libwkv entry point returned a non-zero wkv_status."""

    def __init__(self, fn: str, status: int, hip_error: int = 0):
        self.status = status
        self.hip_error = hip_error
        msg = f"{fn} failed: {wkv_status_string(status)}"
        if hip_error:
            msg += f" (hipError_t {hip_error})"
        super().__init__(msg)


def load_library() -> ctypes.CDLL:
    """Load libwkv.so (built by wkv_recurrence_scan_amd.build) once."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBRARY_PATH):
        raise RuntimeError(
            f"{LIBRARY_PATH} is missing: build it with "
            "`python -m wkv_recurrence_scan_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIBRARY_PATH)
    i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    sigs = {
        "wkv_forward": [i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp],
        "wkv_forward_bf16": [i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp],
        "wkv_forward_ex": [i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, ci, ci, vp],
        "wkv_forward_ws": [i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, ci, ci, vp, i64, vp],
        "wkv_workspace_size": [i64, i64, i64, ci, ci],
        "wkv_workspace_status": [vp, i64, ci, vp],
        "wkv_forward_noalloc": [i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, ci, ci, vp],
        "wkv_token_shift": [i64, i64, i64, i64, vp, vp, vp, vp, vp, ci, vp],
        "wkv_select_path": [i64, i64, i64, ci],
        "wkv_step": [i64, i64, vp, vp, vp, vp, vp, vp, vp],
        "wkv_step_bf16": [i64, i64, vp, vp, vp, vp, vp, vp, vp],
        "wkv_status_string": [ci],
        "wkv_last_hip_error": [],
        "wkv_abi_version": [],
        "wkv_backward": [i64, i64, i64] + [vp] * 15 + [vp, i64, vp],
        "wkv_forward_gated": [i64, i64, i64] + [vp] * 8 + [ci, ci, vp, i64, vp],
        "wkv_step_gated": [i64, i64] + [vp] * 7 + [ci, vp],
        "wkv_backward_workspace_size": [i64, i64, i64],
        "wkv_forward_dd": [i64, i64, i64] + [vp] * 7 + [ci, ci, vp],
        "wkv_step_dd": [i64, i64] + [vp] * 6 + [ci, vp],
        "wkv_matrix_forward": [i64, i64, i64, i64] + [vp] * 8 + [i64, vp],
        "wkv_matrix_workspace_size": [i64, i64, i64, i64],
        "wkv_matrix_step": [i64, i64, i64] + [vp] * 6 + [vp],
        "wkv_ckpt_bytes": [i64, i64, i64],
        "wkv_backward_dd": [i64, i64, i64] + [vp] * 13 + [vp, i64, vp],
        "wkv_backward_dd_workspace_size": [i64, i64, i64],
        "wkv_forward_dd_ckpt": [i64, i64, i64] + [vp] * 8 + [ci, vp],
        "wkv_backward_dd_ckpt": [i64, i64, i64] + [vp] * 14 + [vp, i64, vp],
        "wkv_forward_ckpt": [i64, i64, i64] + [vp] * 9 + [ci, vp],
        "wkv_backward_ckpt": [i64, i64, i64] + [vp] * 16 + [vp, i64, vp],
    }
    for name, args in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = {"wkv_status_string": ctypes.c_char_p,
                      "wkv_workspace_size": ctypes.c_int64,
                      "wkv_backward_workspace_size": ctypes.c_int64,
                      "wkv_ckpt_bytes": ctypes.c_int64,
                      "wkv_backward_dd_workspace_size": ctypes.c_int64,
                      "wkv_matrix_workspace_size": ctypes.c_int64}.get(name, ctypes.c_int)
    if lib.wkv_abi_version() != 1:
        raise RuntimeError(f"{LIBRARY_PATH}: unexpected ABI version {lib.wkv_abi_version()}")
    _lib = lib
    return lib


def wkv_status_string(status: int) -> str:
    return load_library().wkv_status_string(int(status)).decode()


def wkv_abi_version() -> int:
    return load_library().wkv_abi_version()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(device: torch.device, stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, shape, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check(status: int, fn: str):
    if status != 0:
        raise WKVError(fn, status, load_library().wkv_last_hip_error())


def wkv_workspace_size(B: int, T: int, C: int, io: int = WKV_IO_F32, path: str = "auto") -> int:
    """Bytes of workspace wkv_forward_ws needs (0 when the chosen kernel uses none)."""
    r = load_library().wkv_workspace_size(B, T, C, io, _PATHS[path])
    if r < 0:
        raise WKVError("wkv_workspace_size", -r)
    return int(r)


WKV_ERR_LOOKBACK = 9


def wkv_workspace_status(workspace: torch.Tensor, clear: bool = False, stream=None) -> int:
    """wkv_workspace_status: waits for `stream` (default: the current one) and
    returns 0 if no look-back launch with this workspace failed to chain its
    segments since its error word was last cleared, WKV_ERR_LOOKBACK if one did
    (clear=True then resets the word). Other codes raise WKVError."""
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor")
    with torch.cuda.device(workspace.device):
        strm = torch.cuda.current_stream(workspace.device) if stream is None else stream
        st = load_library().wkv_workspace_status(_ptr(workspace), workspace.numel(), int(clear),
                                                 ctypes.c_void_p(strm.cuda_stream))
    if st not in (0, WKV_ERR_LOOKBACK):
        _check(st, "wkv_workspace_status")
    return st


def check_workspace(workspace: Optional[torch.Tensor], stream=None) -> None:
    """Raises WKVError (and clears the word) if a look-back launch with this
    workspace failed to chain its segments; its outputs past the failure are
    NaN. Synchronises the stream."""
    if workspace is not None and wkv_workspace_status(workspace, True, stream) != 0:
        raise WKVError("wkv_forward_ws", WKV_ERR_LOOKBACK)


def _one_shot_workspace(B, T, C, io, path, dev, strm) -> Optional[torch.Tensor]:
    """The workspace a one-shot call takes from the per-(stream, sizes) cache.
    Its status is checked after the call, which synchronises the stream; a
    stream capturing a HIP graph cannot be synchronised, so there AUTO gets
    no workspace (and picks among the kernels that need none) and an explicit
    LOOKBACK must bring its own workspace."""
    with torch.cuda.stream(strm):
        capturing = torch.cuda.is_current_stream_capturing()
    if capturing:
        if path == "lookback":
            raise ValueError("under HIP graph capture a LOOKBACK call needs a workspace of its "
                             "own (or a ForwardCall), since checking the cached one would "
                             "synchronise the capturing stream")
        return None
    return _cached_workspace(wkv_workspace_size(B, T, C, io, path), dev, strm,
                             (B, T, C, io, path))


def new_workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    """A zero-filled device workspace of at least nbytes (None for 0 bytes).
    torch's allocator returns blocks aligned to at least 256 bytes."""
    if nbytes <= 0:
        return None
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


_ws_cache = {}


def _cached_workspace(nbytes: int, device, stream, shape) -> Optional[torch.Tensor]:
    """Workspace reused by one-shot calls with the same sizes on one stream
    (calls on a stream run in order, so they may share it; its layout depends
    on the sizes, so other sizes get another one)."""
    if nbytes <= 0:
        return None
    key = (device.index, stream.cuda_stream, shape)
    ws = _ws_cache.get(key)
    if ws is None:
        if len(_ws_cache) >= 64:
            _ws_cache.clear()
        ws = new_workspace(nbytes, device)
        _ws_cache[key] = ws
    return ws


def wkv_forward_ws(w, u, k, v, state_in=None, out=None, state_out=None, *, path="auto",
                   workspace=None, want_state=True, stream=None):
    """wkv_forward_ws: wkv_forward_ex with a device workspace (a uint8 tensor from
    new_workspace, zero-filled once before its first use). With workspace=None
    one is taken from a per-(stream, sizes) cache and checked after the call
    (see wkv_forward_ex)."""
    return wkv_forward_ex(w, u, k, v, state_in, out, state_out, path=path, workspace=workspace,
                          want_state=want_state, stream=stream)


def wkv_forward_ex(w: torch.Tensor, u: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                   state_in: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                   state_out: Optional[torch.Tensor] = None, *, path: str = "auto",
                   workspace: Optional[torch.Tensor] = None, want_state: bool = True,
                   stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Prefill over (B, T, C). k, v: float32 or bfloat16 (same dtype; out gets
    it too); w, u: (C,) float32; states: (3, B, C) float32. Returns
    (out, state_out); state_out is None when want_state is False and none was
    given. path: "auto", "seq", "chunk" or "lookback". Calls go through
    wkv_forward_ws, so "auto" may pick the look-back scan; its workspace is
    `workspace` or one cached for the stream. A cached workspace is checked
    after the call (check_workspace: the stream is synchronised and a failed
    look-back chain raises WKVError); a workspace passed in is the caller's to
    check with wkv_workspace_status. Under HIP graph capture no cached
    workspace is used: "auto" then picks a kernel that needs none, and
    "lookback" needs `workspace`."""
    lib = load_library()
    if k.dim() != 3:
        raise ValueError(f"k must be (B, T, C), got shape {tuple(k.shape)}")
    if k.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"k must be float32 or bfloat16, got {k.dtype}")
    if path not in _PATHS:
        raise ValueError(f"path must be one of {sorted(_PATHS)}")
    B, T, C = k.shape
    dev = k.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU device")
    _need(v, "v", k.dtype, (B, T, C), dev)
    _need(w, "w", torch.float32, (C,), dev)
    _need(u, "u", torch.float32, (C,), dev)
    _need(k, "k", k.dtype, (B, T, C), dev)
    if state_in is not None:
        _need(state_in, "state_in", torch.float32, (3, B, C), dev)
    if out is None:
        out = torch.empty((B, T, C), dtype=k.dtype, device=dev)
    _need(out, "out", k.dtype, (B, T, C), dev)
    if state_out is None and want_state:
        state_out = torch.empty((3, B, C), dtype=torch.float32, device=dev)
    if state_out is not None:
        _need(state_out, "state_out", torch.float32, (3, B, C), dev)
    io = WKV_IO_BF16 if k.dtype == torch.bfloat16 else WKV_IO_F32
    with torch.cuda.device(dev):
        strm = torch.cuda.current_stream(dev) if stream is None else stream
        owned = workspace is None
        if owned:
            workspace = _one_shot_workspace(B, T, C, io, path, dev, strm)
        elif workspace.device != dev or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous uint8 tensor on the tensors' device")
        st = lib.wkv_forward_ws(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(state_in),
                                _ptr(out), _ptr(state_out), io, _PATHS[path], _ptr(workspace),
                                0 if workspace is None else workspace.numel(),
                                ctypes.c_void_p(strm.cuda_stream))
        _check(st, "wkv_forward_ws")
        if owned:
            check_workspace(workspace, strm)
    return out, state_out


def wkv_forward(w, u, k, v, state_in=None, out=None, state_out=None, *, want_state=True,
                stream=None):
    """wkv_forward: float32 k, v, out; the kernel is chosen by the library."""
    if k.dtype != torch.float32:
        raise TypeError("wkv_forward takes float32 k, v (use wkv_forward_bf16 for bfloat16)")
    return _forward_fixed("wkv_forward", w, u, k, v, state_in, out, state_out, want_state, stream)


def wkv_forward_bf16(w, u, k, v, state_in=None, out=None, state_out=None, *, want_state=True,
                     stream=None):
    """wkv_forward_bf16: bfloat16 k, v, out; fp32 w, u and state."""
    if k.dtype != torch.bfloat16:
        raise TypeError("wkv_forward_bf16 takes bfloat16 k, v")
    return _forward_fixed("wkv_forward_bf16", w, u, k, v, state_in, out, state_out, want_state,
                          stream)


def _forward_fixed(name, w, u, k, v, state_in, out, state_out, want_state, stream):
    lib = load_library()
    B, T, C = k.shape
    dev = k.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU device")
    for t, nm, dt, shp in ((k, "k", k.dtype, (B, T, C)), (v, "v", k.dtype, (B, T, C)),
                           (w, "w", torch.float32, (C,)), (u, "u", torch.float32, (C,))):
        _need(t, nm, dt, shp, dev)
    if state_in is not None:
        _need(state_in, "state_in", torch.float32, (3, B, C), dev)
    if out is None:
        out = torch.empty((B, T, C), dtype=k.dtype, device=dev)
    _need(out, "out", k.dtype, (B, T, C), dev)
    if state_out is None and want_state:
        state_out = torch.empty((3, B, C), dtype=torch.float32, device=dev)
    if state_out is not None:
        _need(state_out, "state_out", torch.float32, (3, B, C), dev)
    with torch.cuda.device(dev):
        st = getattr(lib, name)(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(state_in),
                                _ptr(out), _ptr(state_out), _stream_handle(dev, stream))
    _check(st, name)
    return out, state_out


def _step_fixed(name, dtype, w, u, k, v, state, out, stream):
    lib = load_library()
    if k.dim() != 2:
        raise ValueError(f"k must be (B, C), got shape {tuple(k.shape)}")
    B, C = k.shape
    dev = k.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU device")
    for t, nm, dt, shp in ((k, "k", dtype, (B, C)), (v, "v", dtype, (B, C)),
                           (w, "w", torch.float32, (C,)), (u, "u", torch.float32, (C,)),
                           (state, "state", torch.float32, (3, B, C))):
        _need(t, nm, dt, shp, dev)
    if out is None:
        out = torch.empty((B, C), dtype=dtype, device=dev)
    _need(out, "out", dtype, (B, C), dev)
    with torch.cuda.device(dev):
        st = getattr(lib, name)(B, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(state), _ptr(out),
                                _stream_handle(dev, stream))
    _check(st, name)
    return out


def wkv_step(w, u, k, v, state, out=None, *, stream=None) -> torch.Tensor:
    """wkv_step: one float32 token per sequence, (B, C); state (3, B, C) is
    updated in place. Returns out (B, C)."""
    return _step_fixed("wkv_step", torch.float32, w, u, k, v, state, out, stream)


def wkv_step_bf16(w, u, k, v, state, out=None, *, stream=None) -> torch.Tensor:
    """wkv_step_bf16: bfloat16 k, v, out; fp32 state updated in place."""
    return _step_fixed("wkv_step_bf16", torch.bfloat16, w, u, k, v, state, out, stream)


def wkv_select_path(B: int, T: int, C: int, io: int = WKV_IO_F32) -> str:
    """Name of the kernel the library's automatic choice uses for these sizes
    on the current device when a workspace is available: "seq", "chunk" or
    "lookback" (without a workspace, "lookback" becomes "chunk")."""
    r = load_library().wkv_select_path(B, T, C, io)
    if r < 0:
        raise WKVError("wkv_select_path", -r)
    return _PATH_NAMES[r]


def wkv_backward_workspace_size(B: int, T: int, C: int) -> int:
    """Bytes of workspace wkv_backward needs."""
    r = load_library().wkv_backward_workspace_size(B, T, C)
    if r < 0:
        raise WKVError("wkv_backward_workspace_size", -r)
    return int(r)


def wkv_backward(w: torch.Tensor, u: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                 gout: torch.Tensor, state_in: Optional[torch.Tensor] = None,
                 state_out: Optional[torch.Tensor] = None,
                 gstate_out: Optional[torch.Tensor] = None, *, r: Optional[torch.Tensor] = None,
                 want_gstate_in: bool = True, workspace: Optional[torch.Tensor] = None, out=None,
                 ckpt: Optional[torch.Tensor] = None, stream=None):
    """Gradients of the prefill (float32). Returns (gw, gu, gk, gv, gstate_in)
    for the upstream gradient gout of out (and gstate_out of state_out, which
    must then be the state the forward returned), or (gw, gu, gk, gv,
    gstate_in, gr) when r, the receptance of a gated output, is given.
    gstate_in is None when want_gstate_in is False. `out` may hold
    preallocated (gk, gv, gw, gu, gstate_in[, gr]) tensors; `workspace` a uint8
    tensor of at least wkv_backward_workspace_size bytes (else one is
    allocated for the call). `ckpt`: the checkpoints wkv_forward_ckpt saved
    for the same inputs (wkv_backward_ckpt), or None."""
    lib = load_library()
    if k.dim() != 3:
        raise ValueError(f"k must be (B, T, C), got shape {tuple(k.shape)}")
    B, T, C = k.shape
    dev = k.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU device")
    f32 = torch.float32
    for name, t in (("k", k), ("v", v), ("gout", gout)):
        _need(t, name, f32, (B, T, C), dev)
    if r is not None:
        _need(r, "r", f32, (B, T, C), dev)
    _need(w, "w", f32, (C,), dev)
    _need(u, "u", f32, (C,), dev)
    for name, t in (("state_in", state_in), ("state_out", state_out), ("gstate_out", gstate_out)):
        if t is not None:
            _need(t, name, f32, (3, B, C), dev)
    if out is None:
        gk = torch.empty((B, T, C), dtype=f32, device=dev)
        gv = torch.empty((B, T, C), dtype=f32, device=dev)
        gw = torch.empty((C,), dtype=f32, device=dev)
        gu = torch.empty((C,), dtype=f32, device=dev)
        gs = torch.empty((3, B, C), dtype=f32, device=dev) if want_gstate_in else None
        gr = torch.empty((B, T, C), dtype=f32, device=dev) if r is not None else None
    else:
        gk, gv, gw, gu, gs = out[:5]
        gr = out[5] if len(out) > 5 else None
    for name, t, shape in (("gk", gk, (B, T, C)), ("gv", gv, (B, T, C)), ("gw", gw, (C,)),
                           ("gu", gu, (C,))):
        _need(t, name, f32, shape, dev)
    if gs is not None:
        _need(gs, "gstate_in", f32, (3, B, C), dev)
    if r is not None:
        if gr is None:
            raise ValueError("a gated backward needs a tensor for dL/dr")
        _need(gr, "gr", f32, (B, T, C), dev)
    with torch.cuda.device(dev):
        strm = torch.cuda.current_stream(dev) if stream is None else stream
        nbytes = wkv_backward_workspace_size(B, T, C)
        if workspace is None:
            workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
        elif workspace.device != dev or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous uint8 tensor on the tensors' device")
        if ckpt is None:
            st = lib.wkv_backward(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(r),
                                  _ptr(state_in), _ptr(state_out), _ptr(gstate_out), _ptr(gout),
                                  _ptr(gk), _ptr(gv), _ptr(gr), _ptr(gw), _ptr(gu), _ptr(gs),
                                  _ptr(workspace), workspace.numel(),
                                  ctypes.c_void_p(strm.cuda_stream))
            _check(st, "wkv_backward")
        else:
            _need(ckpt, "ckpt", f32, ckpt_shape(B, T, C), dev)
            st = lib.wkv_backward_ckpt(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(r),
                                       _ptr(state_in), _ptr(state_out), _ptr(gstate_out),
                                       _ptr(gout), _ptr(ckpt), _ptr(gk), _ptr(gv), _ptr(gr),
                                       _ptr(gw), _ptr(gu), _ptr(gs), _ptr(workspace),
                                       workspace.numel(), ctypes.c_void_p(strm.cuda_stream))
            _check(st, "wkv_backward_ckpt")
    return (gw, gu, gk, gv, gs) if r is None else (gw, gu, gk, gv, gs, gr)


CKPT_TOKENS = 8


def ckpt_shape(B: int, T: int, C: int):
    """Shape of the checkpoint tensor (float32): (ceil(T / 8), B, C, 4), the
    lane state (num, den, base, age) in front of every chunk of 8 tokens."""
    return ((T + CKPT_TOKENS - 1) // CKPT_TOKENS, B, C, 4)


def wkv_ckpt_bytes(B: int, T: int, C: int) -> int:
    """Bytes of the checkpoints wkv_forward_ckpt saves for these sizes."""
    n = load_library().wkv_ckpt_bytes(B, T, C)
    if n < 0:
        raise WKVError("wkv_ckpt_bytes", -n)
    return int(n)


def wkv_forward_ckpt(w, u, k, v, r=None, state_in=None, out=None, state_out=None, ckpt=None, *,
                     path="auto", want_state=True, stream=None):
    """wkv_forward_ckpt: the float32 prefill (gated when r is given) that also
    saves the backward pass's checkpoints. Returns (out, state_out, ckpt);
    pass ckpt to wkv_backward(..., ckpt=ckpt) with the same inputs."""
    lib = load_library()
    if k.dim() != 3:
        raise ValueError(f"k must be (B, T, C), got shape {tuple(k.shape)}")
    if path not in ("auto", "seq", "chunk"):
        raise ValueError("path must be 'auto', 'seq' or 'chunk'")
    B, T, C = k.shape
    dev = k.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU device")
    f32 = torch.float32
    for name, t, shape in (("k", k, (B, T, C)), ("v", v, (B, T, C)), ("w", w, (C,)),
                           ("u", u, (C,))):
        _need(t, name, f32, shape, dev)
    if r is not None:
        _need(r, "r", f32, (B, T, C), dev)
    if state_in is not None:
        _need(state_in, "state_in", f32, (3, B, C), dev)
    if out is None:
        out = torch.empty((B, T, C), dtype=f32, device=dev)
    _need(out, "out", f32, (B, T, C), dev)
    if state_out is None and want_state:
        state_out = torch.empty((3, B, C), dtype=f32, device=dev)
    if state_out is not None:
        _need(state_out, "state_out", f32, (3, B, C), dev)
    if ckpt is None:
        ckpt = torch.empty(ckpt_shape(B, T, C), dtype=f32, device=dev)
    _need(ckpt, "ckpt", f32, ckpt_shape(B, T, C), dev)
    with torch.cuda.device(dev):
        st = lib.wkv_forward_ckpt(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(r),
                                  _ptr(state_in), _ptr(out), _ptr(state_out), _ptr(ckpt),
                                  _PATHS[path], _stream_handle(dev, stream))
    _check(st, "wkv_forward_ckpt")
    return out, state_out, ckpt


def wkv_forward_gated(w, u, k, v, r, state_in=None, out=None, state_out=None, *, path="auto",
                      workspace=None, want_state=True, stream=None):
    """wkv_forward_gated: out = sigmoid(r) * wkv, r shaped and typed like k
    (float32 or bfloat16). Returns (out, state_out) like wkv_forward_ex; the
    state is the ungated one."""
    lib = load_library()
    if k.dim() != 3:
        raise ValueError(f"k must be (B, T, C), got shape {tuple(k.shape)}")
    if path not in _PATHS:
        raise ValueError(f"path must be one of {sorted(_PATHS)}")
    B, T, C = k.shape
    dev = k.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU device")
    if k.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"k must be float32 or bfloat16, got {k.dtype}")
    for name, t in (("v", v), ("r", r)):
        _need(t, name, k.dtype, (B, T, C), dev)
    _need(w, "w", torch.float32, (C,), dev)
    _need(u, "u", torch.float32, (C,), dev)
    if state_in is not None:
        _need(state_in, "state_in", torch.float32, (3, B, C), dev)
    if out is None:
        out = torch.empty((B, T, C), dtype=k.dtype, device=dev)
    _need(out, "out", k.dtype, (B, T, C), dev)
    if state_out is None and want_state:
        state_out = torch.empty((3, B, C), dtype=torch.float32, device=dev)
    if state_out is not None:
        _need(state_out, "state_out", torch.float32, (3, B, C), dev)
    io = WKV_IO_BF16 if k.dtype == torch.bfloat16 else WKV_IO_F32
    with torch.cuda.device(dev):
        strm = torch.cuda.current_stream(dev) if stream is None else stream
        owned = workspace is None
        if owned:
            workspace = _one_shot_workspace(B, T, C, io, path, dev, strm)
        st = lib.wkv_forward_gated(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(r),
                                   _ptr(state_in), _ptr(out), _ptr(state_out), io, _PATHS[path],
                                   _ptr(workspace), 0 if workspace is None else workspace.numel(),
                                   ctypes.c_void_p(strm.cuda_stream))
        _check(st, "wkv_forward_gated")
        if owned:
            check_workspace(workspace, strm)
    return out, state_out


def wkv_step_gated(w, u, k, v, r, state, out=None, stream=None):
    """wkv_step_gated: one decode step with out = sigmoid(r) * wkv; k, v, r,
    out (B, C) float32 or bfloat16; the fp32 state is updated in place."""
    lib = load_library()
    B, C = k.shape
    dev = k.device
    for name, t in (("v", v), ("r", r)):
        _need(t, name, k.dtype, (B, C), dev)
    _need(w, "w", torch.float32, (C,), dev)
    _need(u, "u", torch.float32, (C,), dev)
    _need(state, "state", torch.float32, (3, B, C), dev)
    if out is None:
        out = torch.empty((B, C), dtype=k.dtype, device=dev)
    io = WKV_IO_BF16 if k.dtype == torch.bfloat16 else WKV_IO_F32
    with torch.cuda.device(dev):
        st = lib.wkv_step_gated(B, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(r), _ptr(state),
                                _ptr(out), io, _stream_handle(dev, stream))
    _check(st, "wkv_step_gated")
    return out


def wkv_backward_dd_workspace_size(B: int, T: int, C: int) -> int:
    """Bytes of workspace wkv_backward_dd needs."""
    r = load_library().wkv_backward_dd_workspace_size(B, T, C)
    if r < 0:
        raise WKVError("wkv_backward_dd_workspace_size", -r)
    return int(r)


def wkv_backward_dd(w, u, k, v, gout, state_in=None, state_out=None, gstate_out=None, *,
                    want_gstate_in=True, workspace=None, out=None, ckpt=None, stream=None):
    """Gradients of the per-token-decay prefill (float32): returns
    (gw, gu, gk, gv, gstate_in) with gw shaped like w (B, T, C), gu (C,)
    summed over the batch, gstate_in None when want_gstate_in is False.
    `out` may hold preallocated (gk, gv, gw, gu, gstate_in) tensors;
    `workspace` a uint8 tensor of at least wkv_backward_dd_workspace_size
    bytes (else one is allocated for the call). `ckpt`: the checkpoints
    wkv_forward_dd_ckpt saved for the same inputs (wkv_backward_dd_ckpt), or
    None."""
    lib = load_library()
    if k.dim() != 3:
        raise ValueError(f"k must be (B, T, C), got shape {tuple(k.shape)}")
    B, T, C = k.shape
    dev = k.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU device")
    f32 = torch.float32
    for name, t in (("w", w), ("k", k), ("v", v), ("gout", gout)):
        _need(t, name, f32, (B, T, C), dev)
    _need(u, "u", f32, (C,), dev)
    for name, t in (("state_in", state_in), ("state_out", state_out), ("gstate_out", gstate_out)):
        if t is not None:
            _need(t, name, f32, (3, B, C), dev)
    if out is None:
        gk, gv, gw = (torch.empty((B, T, C), dtype=f32, device=dev) for _ in range(3))
        gu = torch.empty((C,), dtype=f32, device=dev)
        gs = torch.empty((3, B, C), dtype=f32, device=dev) if want_gstate_in else None
    else:
        gk, gv, gw, gu, gs = out
    for name, t, shape in (("gk", gk, (B, T, C)), ("gv", gv, (B, T, C)), ("gw", gw, (B, T, C)),
                           ("gu", gu, (C,))):
        _need(t, name, f32, shape, dev)
    if gs is not None:
        _need(gs, "gstate_in", f32, (3, B, C), dev)
    with torch.cuda.device(dev):
        strm = torch.cuda.current_stream(dev) if stream is None else stream
        nbytes = wkv_backward_dd_workspace_size(B, T, C)
        if workspace is None:
            workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
        elif workspace.device != dev or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous uint8 tensor on the tensors' device")
        if ckpt is None:
            st = lib.wkv_backward_dd(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v),
                                     _ptr(state_in), _ptr(state_out), _ptr(gstate_out),
                                     _ptr(gout), _ptr(gk), _ptr(gv), _ptr(gw), _ptr(gu), _ptr(gs),
                                     _ptr(workspace), workspace.numel(),
                                     ctypes.c_void_p(strm.cuda_stream))
            _check(st, "wkv_backward_dd")
        else:
            _need(ckpt, "ckpt", f32, ckpt_shape(B, T, C), dev)
            st = lib.wkv_backward_dd_ckpt(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v),
                                          _ptr(state_in), _ptr(state_out), _ptr(gstate_out),
                                          _ptr(gout), _ptr(ckpt), _ptr(gk), _ptr(gv), _ptr(gw),
                                          _ptr(gu), _ptr(gs), _ptr(workspace), workspace.numel(),
                                          ctypes.c_void_p(strm.cuda_stream))
            _check(st, "wkv_backward_dd_ckpt")
    return gw, gu, gk, gv, gs


def wkv_forward_dd_ckpt(w, u, k, v, state_in=None, out=None, state_out=None, ckpt=None, *,
                        path="auto", want_state=True, stream=None):
    """wkv_forward_dd_ckpt: the float32 per-token-decay prefill that also
    saves the backward's checkpoints. Returns (out, state_out, ckpt); ckpt is
    a float32 tensor of ckpt_shape(B, T, C) holding 16-byte records (num, den
    and a float64 max_exp); pass it to wkv_backward_dd(..., ckpt=ckpt)."""
    lib = load_library()
    if k.dim() != 3:
        raise ValueError(f"k must be (B, T, C), got shape {tuple(k.shape)}")
    if path not in ("auto", "seq", "chunk"):
        raise ValueError("path must be 'auto', 'seq' or 'chunk'")
    B, T, C = k.shape
    dev = k.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU device")
    f32 = torch.float32
    for name, t in (("w", w), ("k", k), ("v", v)):
        _need(t, name, f32, (B, T, C), dev)
    _need(u, "u", f32, (C,), dev)
    if state_in is not None:
        _need(state_in, "state_in", f32, (3, B, C), dev)
    if out is None:
        out = torch.empty((B, T, C), dtype=f32, device=dev)
    _need(out, "out", f32, (B, T, C), dev)
    if state_out is None and want_state:
        state_out = torch.empty((3, B, C), dtype=f32, device=dev)
    if state_out is not None:
        _need(state_out, "state_out", f32, (3, B, C), dev)
    if ckpt is None:
        ckpt = torch.empty(ckpt_shape(B, T, C), dtype=f32, device=dev)
    _need(ckpt, "ckpt", f32, ckpt_shape(B, T, C), dev)
    with torch.cuda.device(dev):
        st = lib.wkv_forward_dd_ckpt(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(state_in),
                                     _ptr(out), _ptr(state_out), _ptr(ckpt), _PATHS[path],
                                     _stream_handle(dev, stream))
    _check(st, "wkv_forward_dd_ckpt")
    return out, state_out, ckpt


def wkv_forward_dd(w, u, k, v, state_in=None, out=None, state_out=None, *, path="auto",
                   want_state=True, stream=None):
    """wkv_forward_dd: prefill with a per-token decay. w, k, v: (B, T, C) of one
    dtype (float32 or bfloat16; out gets it too), w > 0 the rate of each step;
    u: (C,) float32; states (3, B, C) float32. path: "auto", "seq" or "chunk".
    Returns (out, state_out)."""
    lib = load_library()
    if k.dim() != 3:
        raise ValueError(f"k must be (B, T, C), got shape {tuple(k.shape)}")
    if k.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"k must be float32 or bfloat16, got {k.dtype}")
    if path not in ("auto", "seq", "chunk"):
        raise ValueError("path must be one of auto, seq, chunk")
    B, T, C = k.shape
    dev = k.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU device")
    for name, t in (("v", v), ("w", w)):
        _need(t, name, k.dtype, (B, T, C), dev)
    _need(u, "u", torch.float32, (C,), dev)
    if state_in is not None:
        _need(state_in, "state_in", torch.float32, (3, B, C), dev)
    if out is None:
        out = torch.empty((B, T, C), dtype=k.dtype, device=dev)
    _need(out, "out", k.dtype, (B, T, C), dev)
    if state_out is None and want_state:
        state_out = torch.empty((3, B, C), dtype=torch.float32, device=dev)
    if state_out is not None:
        _need(state_out, "state_out", torch.float32, (3, B, C), dev)
    io = WKV_IO_BF16 if k.dtype == torch.bfloat16 else WKV_IO_F32
    with torch.cuda.device(dev):
        st = lib.wkv_forward_dd(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(state_in),
                                _ptr(out), _ptr(state_out), io, _PATHS[path],
                                _stream_handle(dev, stream))
    _check(st, "wkv_forward_dd")
    return out, state_out


def wkv_step_dd(w, u, k, v, state, out=None, *, stream=None):
    """wkv_step_dd: one decode step with this step's rates w; w, k, v, out (B, C)
    of one dtype (float32 or bfloat16); u (C,) float32; the fp32 state (3, B, C)
    is updated in place. Returns out."""
    lib = load_library()
    if k.dim() != 2:
        raise ValueError(f"k must be (B, C), got shape {tuple(k.shape)}")
    B, C = k.shape
    dev = k.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU device")
    for name, t in (("v", v), ("w", w)):
        _need(t, name, k.dtype, (B, C), dev)
    _need(u, "u", torch.float32, (C,), dev)
    _need(state, "state", torch.float32, (3, B, C), dev)
    if out is None:
        out = torch.empty((B, C), dtype=k.dtype, device=dev)
    _need(out, "out", k.dtype, (B, C), dev)
    io = WKV_IO_BF16 if k.dtype == torch.bfloat16 else WKV_IO_F32
    with torch.cuda.device(dev):
        st = lib.wkv_step_dd(B, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(state), _ptr(out), io,
                             _stream_handle(dev, stream))
    _check(st, "wkv_step_dd")
    return out


MATRIX_HEAD = 64


def wkv_matrix_workspace_size(B: int, T: int, H: int, D: int = MATRIX_HEAD) -> int:
    """Bytes of workspace that lets wkv_matrix_forward use all its segments."""
    r = load_library().wkv_matrix_workspace_size(B, T, H, D)
    if r < 0:
        raise WKVError("wkv_matrix_workspace_size", -r)
    return int(r)


def wkv_matrix_forward(w, k, v, r, H: int, state_in=None, out=None, state_out=None, *,
                       workspace="auto", want_state=True, stream=None):
    """wkv_matrix_forward: the matrix-valued-state recurrence over (B, T, C),
    C = H * 64, float32. w: positive decay rates; k, v, r: key, value,
    receptance, all (B, T, C); states (B, H, 64, 64). workspace: a uint8
    tensor, None (no segments) or "auto" (one of wkv_matrix_workspace_size
    bytes, allocated for the call). Returns (out, state_out)."""
    lib = load_library()
    if k.dim() != 3:
        raise ValueError(f"k must be (B, T, C), got shape {tuple(k.shape)}")
    B, T, C = k.shape
    if H <= 0 or C != H * MATRIX_HEAD:
        raise ValueError(f"C = {C} must be H * {MATRIX_HEAD} with H = {H}")
    dev = k.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU device")
    f32 = torch.float32
    for name, t in (("w", w), ("k", k), ("v", v), ("r", r)):
        _need(t, name, f32, (B, T, C), dev)
    sshape = (B, H, MATRIX_HEAD, MATRIX_HEAD)
    if state_in is not None:
        _need(state_in, "state_in", f32, sshape, dev)
    if out is None:
        out = torch.empty((B, T, C), dtype=f32, device=dev)
    _need(out, "out", f32, (B, T, C), dev)
    if state_out is None and want_state:
        state_out = torch.empty(sshape, dtype=f32, device=dev)
    if state_out is not None:
        _need(state_out, "state_out", f32, sshape, dev)
    with torch.cuda.device(dev):
        if isinstance(workspace, str):
            n = wkv_matrix_workspace_size(B, T, H)
            workspace = torch.empty(n, dtype=torch.uint8, device=dev) if n > 0 else None
        elif workspace is not None and (workspace.device != dev or workspace.dtype != torch.uint8
                                        or not workspace.is_contiguous()):
            raise ValueError("workspace must be a contiguous uint8 tensor on the tensors' device")
        st = lib.wkv_matrix_forward(B, T, H, MATRIX_HEAD, _ptr(w), _ptr(k), _ptr(v), _ptr(r),
                                    _ptr(state_in), _ptr(out), _ptr(state_out), _ptr(workspace),
                                    0 if workspace is None else workspace.numel(),
                                    _stream_handle(dev, stream))
    _check(st, "wkv_matrix_forward")
    return out, state_out


def wkv_matrix_step(w, k, v, r, H: int, state, out=None, *, stream=None):
    """wkv_matrix_step: one token (B, C) of the matrix-valued-state recurrence;
    the state (B, H, 64, 64) is updated in place. Returns out (B, C)."""
    lib = load_library()
    if k.dim() != 2:
        raise ValueError(f"k must be (B, C), got shape {tuple(k.shape)}")
    B, C = k.shape
    if H <= 0 or C != H * MATRIX_HEAD:
        raise ValueError(f"C = {C} must be H * {MATRIX_HEAD} with H = {H}")
    dev = k.device
    f32 = torch.float32
    for name, t in (("w", w), ("k", k), ("v", v), ("r", r)):
        _need(t, name, f32, (B, C), dev)
    _need(state, "state", f32, (B, H, MATRIX_HEAD, MATRIX_HEAD), dev)
    if out is None:
        out = torch.empty((B, C), dtype=f32, device=dev)
    _need(out, "out", f32, (B, C), dev)
    with torch.cuda.device(dev):
        st = lib.wkv_matrix_step(B, H, MATRIX_HEAD, _ptr(w), _ptr(k), _ptr(v), _ptr(r),
                                 _ptr(state), _ptr(out), _stream_handle(dev, stream))
    _check(st, "wkv_matrix_step")
    return out


def wkv_token_shift(mu: torch.Tensor, x: torch.Tensor, x_prev: Optional[torch.Tensor] = None,
                    out: Optional[torch.Tensor] = None, x_last: Optional[torch.Tensor] = None, *,
                    want_last: bool = True, stream=None):
    """wkv_token_shift: mu (P, C) float32; x (B, T, C) float32 or bfloat16;
    x_prev (B, C) like x or None (zeros). Returns (out (P, B, T, C), x_last
    (B, C) or None); x_last may be x_prev itself (updated in place)."""
    lib = load_library()
    if x.dim() != 3:
        raise ValueError(f"x must be (B, T, C), got shape {tuple(x.shape)}")
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"x must be float32 or bfloat16, got {x.dtype}")
    B, T, C = x.shape
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU device")
    if mu.dim() != 2:
        raise ValueError(f"mu must be (P, C), got shape {tuple(mu.shape)}")
    P = mu.shape[0]
    _need(mu, "mu", torch.float32, (P, C), dev)
    _need(x, "x", x.dtype, (B, T, C), dev)
    if x_prev is not None:
        _need(x_prev, "x_prev", x.dtype, (B, C), dev)
    if out is None:
        out = torch.empty((P, B, T, C), dtype=x.dtype, device=dev)
    _need(out, "out", x.dtype, (P, B, T, C), dev)
    if x_last is None and want_last:
        x_last = torch.empty((B, C), dtype=x.dtype, device=dev)
    if x_last is not None:
        _need(x_last, "x_last", x.dtype, (B, C), dev)
    io = WKV_IO_BF16 if x.dtype == torch.bfloat16 else WKV_IO_F32
    with torch.cuda.device(dev):
        st = lib.wkv_token_shift(B, T, C, P, _ptr(mu), _ptr(x), _ptr(x_prev), _ptr(out),
                                 _ptr(x_last), io, _stream_handle(dev, stream))
    _check(st, "wkv_token_shift")
    return out, x_last


class ForwardCall:
    """A wkv_forward_ws call validated once and launched many times.

    The tensors are checked (device, dtype, shape, contiguity) and their
    pointers captured at construction; each call then only passes the saved
    arguments and the stream to the C entry point. Keep the tensors alive and
    unmoved while the object is used. Useful in per-layer loops and under HIP
    graph capture, where per-call Python checks would dominate a ~10 us kernel.
    The object owns the workspace of its kernel (zero-filled once here), so
    two ForwardCall objects may run on different streams at the same time.
    """

    def __init__(self, w, u, k, v, state_in=None, out=None, state_out=None, *, path="auto",
                 want_state=True):
        if k.dim() != 3:
            raise ValueError(f"k must be (B, T, C), got shape {tuple(k.shape)}")
        if k.dtype not in (torch.float32, torch.bfloat16):
            raise TypeError(f"k must be float32 or bfloat16, got {k.dtype}")
        if path not in _PATHS:
            raise ValueError(f"path must be one of {sorted(_PATHS)}")
        B, T, C = k.shape
        dev = k.device
        if dev.type != "cuda":
            raise ValueError("tensors must live on a GPU device")
        for t, nm, dt, shp in ((k, "k", k.dtype, (B, T, C)), (v, "v", k.dtype, (B, T, C)),
                               (w, "w", torch.float32, (C,)), (u, "u", torch.float32, (C,))):
            _need(t, nm, dt, shp, dev)
        if state_in is not None:
            _need(state_in, "state_in", torch.float32, (3, B, C), dev)
        if out is None:
            out = torch.empty((B, T, C), dtype=k.dtype, device=dev)
        _need(out, "out", k.dtype, (B, T, C), dev)
        if state_out is None and want_state:
            state_out = torch.empty((3, B, C), dtype=torch.float32, device=dev)
        if state_out is not None:
            _need(state_out, "state_out", torch.float32, (3, B, C), dev)
        self.device = dev
        self.out, self.state_out = out, state_out
        io = WKV_IO_BF16 if k.dtype == torch.bfloat16 else WKV_IO_F32
        with torch.cuda.device(dev):
            self.workspace = new_workspace(wkv_workspace_size(B, T, C, io, path), dev)
        self._keep = (w, u, k, v, state_in)
        self._fn = load_library().wkv_forward_ws
        ws_bytes = 0 if self.workspace is None else self.workspace.numel()
        self._args = (B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(state_in), _ptr(out),
                      _ptr(state_out), io, _PATHS[path], _ptr(self.workspace), ws_bytes)

    def __call__(self, stream=None):
        s = torch.cuda.current_stream(self.device) if stream is None else stream
        st = self._fn(*self._args, ctypes.c_void_p(s.cuda_stream))
        if st != 0:
            _check(st, "wkv_forward_ws")
        return self.out, self.state_out

    def check(self, stream=None) -> None:
        """Raises WKVError if a look-back launch of this call failed to chain
        its segments since the last check (synchronises the stream)."""
        check_workspace(self.workspace, stream)


class StepCall:
    """A wkv_step / wkv_step_bf16 call validated once and launched many times
    (the decode loop's per-token launch, without per-call Python checks).
    Keep the tensors alive and unmoved while the object is used."""

    def __init__(self, w, u, k, v, state, out=None):
        if k.dim() != 2:
            raise ValueError(f"k must be (B, C), got shape {tuple(k.shape)}")
        if k.dtype not in (torch.float32, torch.bfloat16):
            raise TypeError(f"k must be float32 or bfloat16, got {k.dtype}")
        B, C = k.shape
        dev = k.device
        if dev.type != "cuda":
            raise ValueError("tensors must live on a GPU device")
        if out is None:
            out = torch.empty((B, C), dtype=k.dtype, device=dev)
        for t, nm, dt, shp in ((k, "k", k.dtype, (B, C)), (v, "v", k.dtype, (B, C)),
                               (w, "w", torch.float32, (C,)), (u, "u", torch.float32, (C,)),
                               (state, "state", torch.float32, (3, B, C)),
                               (out, "out", k.dtype, (B, C))):
            _need(t, nm, dt, shp, dev)
        self.device = dev
        self.out = out
        self._keep = (w, u, k, v, state)
        lib = load_library()
        self._name = "wkv_step_bf16" if k.dtype == torch.bfloat16 else "wkv_step"
        self._fn = getattr(lib, self._name)
        self._args = (B, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(state), _ptr(out))

    def __call__(self, stream=None):
        s = torch.cuda.current_stream(self.device) if stream is None else stream
        st = self._fn(*self._args, ctypes.c_void_p(s.cuda_stream))
        if st != 0:
            _check(st, self._name)
        return self.out


def forward(w, u, k, v, state=None, *, path="auto", out=None, state_out=None):
    """Convenience: prefill for float32 or bfloat16 k, v. Returns (out, state_out)."""
    return wkv_forward_ex(w, u, k, v, state, out, state_out, path=path)


def step(w, u, k, v, state, *, out=None):
    """Convenience: one decode step for float32 or bfloat16 k, v; state in place."""
    if k.dtype == torch.bfloat16:
        return wkv_step_bf16(w, u, k, v, state, out)
    return wkv_step(w, u, k, v, state, out)

"""RWKV weighted-key-value (WKV) operator on AMD MI355X (gfx950).

The work is done by hand-written HIP kernels in libwkv.so behind the C
interface declared in include/wkv.h; this package only marshals torch tensors
into that interface (see _lib). Build the library with
`python -m wkv_recurrence_scan_amd.build`.

    out, state = wkv_forward(w, u, k, v)            # prefill, float32
    out, state = wkv_forward_bf16(w, u, k, v)       # prefill, bfloat16 I/O
    y = wkv_step(w, u, k_t, v_t, state)             # decode, state in place
    gw, gu, gk, gv, gs = wkv_backward(w, u, k, v, gout)  # gradients
    out, state = wkv_forward_dd(w_t, u, k, v)     # per-token decay w_t (B, T, C)
    gw_t, gu, gk, gv, gs = wkv_backward_dd(w_t, u, k, v, gout)  # its gradients
    y, S = wkv_matrix_forward(w_t, k, v, r, H)     # matrix-valued state per head
    xs, x_last = wkv_token_shift(mu, x, x_prev)     # token shift ahead of the projections
    out, state = wkv(w, u, k, v, r=None, state_in=None)  # autograd (checkpointed pair)
"""

from ._lib import (  # noqa: F401
    LIBRARY_PATH,
    MATRIX_HEAD,
    WKV_IO_BF16,
    WKV_IO_F32,
    WKV_PATH_AUTO,
    WKV_PATH_CHUNK,
    WKV_PATH_LOOKBACK,
    WKV_PATH_SEQ,
    ForwardCall,
    StepCall,
    WKV_ERR_LOOKBACK,
    WKVError,
    check_workspace,
    forward,
    load_library,
    new_workspace,
    step,
    wkv_abi_version,
    wkv_backward,
    wkv_backward_dd,
    wkv_backward_dd_workspace_size,
    wkv_forward_ckpt,
    wkv_ckpt_bytes,
    ckpt_shape,
    CKPT_TOKENS,
    wkv_backward_workspace_size,
    wkv_forward,
    wkv_forward_bf16,
    wkv_forward_dd,
    wkv_forward_dd_ckpt,
    wkv_forward_ex,
    wkv_forward_gated,
    wkv_forward_ws,
    wkv_matrix_forward,
    wkv_matrix_step,
    wkv_matrix_workspace_size,
    wkv_select_path,
    wkv_status_string,
    wkv_step,
    wkv_step_bf16,
    wkv_step_dd,
    wkv_step_gated,
    wkv_workspace_size,
    wkv_workspace_status,
    wkv_token_shift,
)
from .autograd import WKVFunction, wkv  # noqa: F401,E402

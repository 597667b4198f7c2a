"""Differentiable float32 prefill for torch.autograd.

The forward runs the library's checkpoint-saving prefill (wkv_forward_ckpt:
the lane state in front of every 8-token chunk, 2 bytes per channel-token)
and the backward reads those checkpoints (wkv_backward with ckpt), so a
training step re-runs no part of the forward scan. The gradients are those of
wkv_backward: dL/dw, dL/du, dL/dk, dL/dv, dL/dr for a gated output and
dL/d(num, den, max_exp) of the initial state.

The final state is a representation (num, den, max_exp) of the sums
num * e^max_exp and den * e^max_exp. Its gradient is taken through num and den
at the returned max_exp, as wkv_backward does: the max_exp plane of the
incoming gradient is not used. The state returned is safe to update in place
afterwards (a decode step does): the backward keeps its own copy.

    out, state = wkv(w, u, k, v)                 # ungated
    y, state = wkv(w, u, k, v, r=r, state_in=s0)   # y = sigmoid(r) * wkv
    (y * g).sum().backward()
"""

from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import _lib


class WKVFunction(torch.autograd.Function):
    """autograd node of the checkpointed prefill (float32 I/O)."""

    @staticmethod
    def forward(ctx, w, u, k, v, r, state_in):
        out, state_out, ckpt = _lib.wkv_forward_ckpt(w, u, k, v, r=r, state_in=state_in)
        ctx.save_for_backward(w, u, k, v, r, state_in, state_out.clone(), ckpt)
        return out, state_out

    @staticmethod
    def backward(ctx, gout, gstate):
        w, u, k, v, r, state_in, state_out, ckpt = ctx.saved_tensors
        gout = torch.zeros_like(k) if gout is None else gout.contiguous()
        gstate = None if gstate is None else gstate.contiguous()
        want_gs = state_in is not None and ctx.needs_input_grad[5]
        res = _lib.wkv_backward(w, u, k, v, gout, state_in=state_in,
                                state_out=state_out if gstate is not None else None,
                                gstate_out=gstate, r=r, want_gstate_in=want_gs, ckpt=ckpt)
        gw, gu, gk, gv, gs = res[:5]
        gr = res[5] if r is not None else None
        return gw, gu, gk, gv, gr, gs


def wkv(w: torch.Tensor, u: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
        r: Optional[torch.Tensor] = None,
        state_in: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """(out, state_out) of the float32 prefill, differentiable in w (C,),
    u (C,), k, v (B, T, C), r (B, T, C; gated output when given) and state_in
    (3, B, C). All tensors contiguous float32 on one GPU."""
    return WKVFunction.apply(w, u, k, v, r, state_in)

"""GPU parity on seeded random sizes: 48 cases drawn once (fixed seed) over
B in [1, 40), T log-uniform in [1, 5000], C log-uniform in [1, 1100] or one of
the kernels' tile widths, B*T*C <= 2e6; element type, operator (plain,
gated, per-token decay), path (AUTO and every explicit kernel the operator
has) and an initial state drawn per case. Each case against the float64
oracle at the tolerances of the other parity tests."""

import numpy as np
import pytest
import torch

from oracle import sigmoid, wkv_dd_recurrent
from wkvtest import (BF16_TOL, F32_TOL, I, W, assert_out_close, assert_state_close, dev_f32,
                     dev_io, host64, make_case, random_state, say, wkv_recurrent)

pytestmark = pytest.mark.gpu

WL3, WL4 = I.WORKLOADS[3], I.WORKLOADS[4]


def _cases(n=48, seed=2024):
    g = np.random.default_rng(seed)
    out = []
    for i in range(n):
        while True:
            B = int(g.integers(1, 40))
            T = int(np.exp(g.uniform(0, np.log(5000))))
            C = int(np.exp(g.uniform(0, np.log(1100))))
            if g.random() < 0.3:
                C = int(g.choice([256, 512, 768, 1024, 64, 96, 2, 4]))
            if B * T * C <= 2_000_000:
                break
        io = "bf16" if g.random() < 0.5 else "f32"
        kind = str(g.choice(["plain", "gated", "dd"]))
        path = str(g.choice(["auto", "seq", "chunk"] + ([] if kind == "dd" else ["lookback"])))
        out.append((i, kind, io, path, B, T, C, bool(g.random() < 0.4)))
    return out


@pytest.mark.parametrize("i,kind,io,path,B,T,C,with_state", _cases(),
                         ids=lambda x: str(x) if not isinstance(x, bool) else ("s" if x else "e"))
def test_random_size(i, kind, io, path, B, T, C, with_state):
    say(f"random case {i}: {kind} {io} path={path} B={B} T={T} C={C} state={with_state}")
    wl = WL4 if io == "bf16" else WL3
    w, u, k, v = make_case(wl, B, T, C, layer=i % 8)
    if io == "bf16":
        k, v = I.round_to_bf16(k), I.round_to_bf16(v)
    s0 = random_state(B, C, 300 + i) if with_state else None
    ds = None if s0 is None else dev_f32(s0)
    s064 = None if s0 is None else s0.astype(np.float64)
    if kind == "dd":
        wt = I.decay_rates(wl.scaled(B=B, T=T, C=C), 0)
        if io == "bf16":
            wt = I.round_to_bf16(wt)
        out, st = W.wkv_forward_dd(dev_io(wt, io), dev_f32(u), dev_io(k, io), dev_io(v, io), ds,
                                   path=path)
        ref, rst = wkv_dd_recurrent(wt, u, k, v, s064)
    elif kind == "gated":
        r = np.random.default_rng([65, i]).normal(0, 2, (B, T, C)).astype(np.float32)
        if io == "bf16":
            r = I.round_to_bf16(r)
        out, st = W.wkv_forward_gated(dev_f32(w), dev_f32(u), dev_io(k, io), dev_io(v, io),
                                      dev_io(r, io), ds, path=path)
        ref, rst = wkv_recurrent(w, u, k, v, s064)
        ref = ref * sigmoid(r)
    else:
        out, st = W.wkv_forward_ex(dev_f32(w), dev_f32(u), dev_io(k, io), dev_io(v, io), ds,
                                   path=path)
        ref, rst = wkv_recurrent(w, u, k, v, s064)
    torch.cuda.synchronize()
    assert_out_close(host64(out), ref, v, BF16_TOL if io == "bf16" else F32_TOL)
    assert_state_close(host64(st), rst, F32_TOL * (10 if io == "bf16" else 1))

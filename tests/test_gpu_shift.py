"""GPU parity of the token shift (wkv_token_shift, through the C interface)
with the float64 oracle (oracle/wkv_shift.py), element by element: ragged
sizes around the 16-byte channel pieces and the 8- and 16-token runs, one to
eight projections, fp32 and bf16, with and without the previous token, the
carried last token in place (decode chain), T = 0, and the MicroRWKV layer
shape in full.

Tolerances: one fused multiply-add in fp32 per element, so fp32 results are
within 1e-6 of the oracle relative to |ref| + rms(x); bf16 results are the
fp32 ones rounded to nearest even, within 2^-8 relative."""

import numpy as np
import pytest
import torch

from oracle.wkv_shift import token_shift
from wkvtest import I, W, dev_io, host64, rms, say

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-6, "bf16": 2.0 ** -8}
WL0, WL4 = I.WORKLOADS[0], I.WORKLOADS[4]


def _close(got, ref, scale, tol, what):
    got = np.asarray(got, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), what
    err = np.abs(got - ref) / (np.abs(ref) + scale)
    assert err.size == 0 or err.max() <= tol, f"{what}: max error {err.max():.3e} > {tol:.1e}"


def _case(io, B, T, C, P, seed=0):
    wl = (WL4 if io == "bf16" else WL0).scaled(B=B, T=T, C=C)
    x, mu, xp = I.shift_inputs(wl, layer=seed, P=P)
    return x, mu, xp


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("B,T,C,P", [(1, 1, 1, 1), (2, 3, 5, 4), (1, 17, 8, 2), (2, 16, 64, 4),
                                     (3, 33, 96, 5), (1, 100, 7, 8), (2, 257, 768, 4),
                                     (1, 9, 24, 3)])
@pytest.mark.parametrize("with_prev", [False, True], ids=["zeros", "prev"])
def test_token_shift_matches_oracle(io, B, T, C, P, with_prev):
    say(f"token shift io={io} B={B} T={T} C={C} P={P} prev={with_prev}")
    x, mu, xp = _case(io, B, T, C, P)
    out, last = W.wkv_token_shift(torch.from_numpy(mu).cuda(), dev_io(x, io),
                                  dev_io(xp, io) if with_prev else None)
    torch.cuda.synchronize()
    ref, rlast = token_shift(x, mu, xp if with_prev else None)
    s = max(rms(x), 1e-30)
    _close(host64(out), ref, s, TOL[io], "mixes")
    assert np.array_equal(host64(last), x[:, -1].astype(np.float64))


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_decode_chain_in_place(io):
    """T one-token calls carrying the last token in place (x_last is x_prev)
    give the one call over all T tokens."""
    B, T, C, P = 3, 12, 40, 4
    say(f"token shift decode chain io={io}")
    x, mu, xp = _case(io, B, T, C, P, seed=1)
    dmu, dx = torch.from_numpy(mu).cuda(), dev_io(x, io)
    carry = dev_io(xp, io)
    steps = []
    for t in range(T):
        o, last = W.wkv_token_shift(dmu, dx[:, t:t + 1].contiguous(), carry, x_last=carry)
        assert last is carry
        steps.append(o)
    full, flast = W.wkv_token_shift(dmu, dx, dev_io(xp, io))
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(steps, dim=2), full)
    assert torch.equal(carry, flast)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_empty_sequence_carries_the_previous_token(io):
    x, mu, xp = _case(io, 2, 0, 16, 2)
    out, last = W.wkv_token_shift(torch.from_numpy(mu).cuda(), dev_io(x, io), dev_io(xp, io))
    out2, last2 = W.wkv_token_shift(torch.from_numpy(mu).cuda(), dev_io(x, io), None)
    torch.cuda.synchronize()
    assert out.shape == (2, 2, 0, 16)
    assert np.array_equal(host64(last), xp.astype(np.float64))
    assert torch.count_nonzero(last2).item() == 0


def test_microrwkv_layer_shape_in_full():
    """The shift in front of the WKV operator at the MicroRWKV layer shape
    (B=8 T=1024 C=768, four projections), every element against the oracle."""
    wl = I.WORKLOADS[1].scaled(layers=1)
    say("token shift at B=8 T=1024 C=768")
    x, mu, xp = I.shift_inputs(wl)
    out, last = W.wkv_token_shift(torch.from_numpy(mu).cuda(), torch.from_numpy(x).cuda(),
                                  torch.from_numpy(xp).cuda())
    torch.cuda.synchronize()
    ref, _ = token_shift(x, mu, xp)
    _close(host64(out), ref, rms(x), TOL["f32"], "mixes")
    assert np.array_equal(host64(last), x[:, -1].astype(np.float64))

"""GPU parity of the self-decoder's SWA layer -- hs2_rope_partial on the
queries and keys, then hs2_swa_attn -- against the float64 oracle: several key
tiles, ragged token blocks, windows from 1 to past the sequence start, rotation
of none, some or all dims, and positions near 2^20 where the angles need more
than float32.  hs2_rope_partial alone is checked element by element.  Rules:
parity.py."""
import os
import sys

import numpy as np
import pytest
import torch

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import parity  # noqa: E402

import oracle  # noqa: E402
from token_level_sparse_full_amd import hs2, inputs  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print("[case]", *a, flush=True)


@pytest.mark.parametrize("B,H,n_q,T,q_pos0,window,rope_dims,base", [
    (1, 16, 70, 500, 430, 128, 64, 10000.0),
    (2, 16, 33, 33, 0, 128, 64, 10000.0),        # windows reaching past the sequence start
    (1, 8, 100, 1200, 1000, 300, 64, 10000.0),
    (2, 4, 129, 700, 0, 5, 8, 100.0),
    (1, 2, 90, 1000, 910, 1, 0, 10000.0),        # window of one, no rotation
    (1, 1, 300, 2000, 1700, 128, 256, 500000.0),  # every dim rotated
    (1, 16, 20, 1 << 20, (1 << 20) - 20, 128, 64, 10000.0),   # positions near 2^20
    (1, 16, 257, 3000, 2743, 64, 64, 10000.0),
])
def test_swa_parity(B, H, n_q, T, q_pos0, window, rope_dims, base):
    say("swa", B, H, n_q, T, q_pos0, window, rope_dims, base)
    inp = inputs.attention_inputs(B=B, n_q=n_q, T=T, H=H, d=256, kv="bf16", n_sparse=0, seed=51, device=DEV)
    qr = torch.stack([hs2.hs2_rope_partial(inp["q"][b], pos0=q_pos0, rope_dims=rope_dims, rope_base=base)
                      for b in range(B)])
    kr = torch.stack([hs2.hs2_rope_partial(inp["k"][b], pos0=0, rope_dims=rope_dims, rope_base=base)
                      for b in range(B)])
    o, lse = hs2.hs2_swa_attn(qr, kr, inp["v"], q_pos0=q_pos0, window=window, sm_scale=1 / 16)
    torch.cuda.synchronize()
    first = max(0, q_pos0 - window + 1)
    for b in range(B):
        k64 = np.zeros((q_pos0 + n_q, 256))
        v64 = np.zeros((q_pos0 + n_q, 256))
        k64[first:] = parity.decode(inp["k"][b, first: q_pos0 + n_q])
        v64[first:] = parity.decode(inp["v"][b, first: q_pos0 + n_q])
        o_ref, lse_ref = oracle.swa_attn(parity.decode(inp["q"][b]), k64, v64, q_pos0, window, rope_dims, base, 1 / 16)
        parity.check_out(o[b], o_ref, "bf16")
        parity.check_lse(lse[b], lse_ref)


def test_swa_deterministic():
    say("swa twice")
    inp = inputs.attention_inputs(B=1, n_q=300, T=900, H=16, d=256, kv="bf16", n_sparse=0, seed=52, device=DEV)
    outs = []
    for fill in (0, 7):
        o = torch.full_like(inp["q"], fill)
        lse = torch.full((1, 300, 16), float(fill), device=DEV)
        hs2.hs2_swa_attn(inp["q"], inp["k"], inp["v"], q_pos0=600, window=128, o=o, lse=lse)
        torch.cuda.synchronize()
        outs.append((o.view(torch.int16).clone(), lse.view(torch.int32).clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def _bf16_ulp(x):
    return 2.0 ** (np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126))) - 7)


@pytest.mark.parametrize("n_pos,heads,pos0,rope_dims,base,inplace", [
    (300, 16, 0, 64, 10000.0, False),
    (257, 1, (1 << 20) - 257, 64, 10000.0, True),
    (100, 4, 123456, 256, 500000.0, False),
    (64, 2, 7, 8, 100.0, True),
    (33, 1, 5, 0, 10000.0, False),
])
def test_rope_partial_parity(n_pos, heads, pos0, rope_dims, base, inplace):
    """Each turned value within one bf16 step of the exactly turned value (half a
    step of rounding, plus the float32 sine and cosine), nearly all of them equal
    to its correct rounding; dims past rope_dims are copied bit for bit."""
    say("rope", n_pos, heads, pos0, rope_dims, base, inplace)
    g = torch.Generator(device=DEV)
    g.manual_seed(n_pos)
    x = (torch.randn((n_pos, heads, 256), generator=g, device=DEV) * 2.0).to(torch.bfloat16)
    x_in = x.clone()
    y = hs2.hs2_rope_partial(x, pos0=pos0, rope_dims=rope_dims, rope_base=base, out=x if inplace else None)
    torch.cuda.synchronize()
    x64 = parity.decode(x_in)
    ref = oracle.rope_partial(np.swapaxes(x64, 0, 1), pos0 + np.arange(n_pos), rope_dims, base)
    ref = np.swapaxes(ref, 0, 1)
    got = parity.decode(y)
    pair_mag = np.repeat(np.abs(x64[..., 0::2]) + np.abs(x64[..., 1::2]), 2, axis=-1)
    err = np.abs(got - ref)
    assert (err <= _bf16_ulp(ref) * 0.5 * (1 + 2.0 ** -7) + pair_mag * 2.0 ** -18).all()
    exact = oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits(ref))
    assert (got == exact).mean() > 0.99
    np.testing.assert_array_equal(inputs.raw_numpy(y)[..., rope_dims:], inputs.raw_numpy(x_in)[..., rope_dims:])

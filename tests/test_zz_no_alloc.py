"""hs2_sparse_attn_reuse_noalloc (static scratch, no allocation) against
hs2_sparse_attn_reuse (caller's workspace) through the C ABI: the same kernels
run in the same order, so the outputs must be equal bit for bit.  Two calls in
a row share the static scratch, the second with a smaller input; the largest
accepted split-form size (1024 (query, piece) slots) and the one-workgroup-
per-query form are covered too.  The first call is also checked against the
oracle."""
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


def _case(B, n_q, T, H, kv, max_sel, seed):
    inp = inputs.attention_inputs(B=B, n_q=n_q, T=T, H=H, d=256, kv=kv, n_sparse=0, seed=seed, device=DEV)
    rng = np.random.default_rng(seed)
    idx = np.full((B, n_q, max_sel), -1, dtype=np.int32)
    cnt = np.zeros((B, n_q), dtype=np.int32)
    sizes = [0, 1, 77, 128, 129, max_sel // 2, max_sel]
    for b in range(B):
        for i in range(n_q):
            n = sizes[(b * n_q + i) % len(sizes)]
            idx[b, i, :n] = np.sort(rng.choice(T, size=n, replace=False))
            cnt[b, i] = n
    return inp, idx, cnt


def _both(inp, idx, cnt):
    idx_t, cnt_t = torch.from_numpy(idx).to(DEV), torch.from_numpy(cnt).to(DEV)
    kw = dict(sm_scale=1 / 16, k_scale=inp["k_scale"], v_scale=inp["v_scale"])
    o_ref, lse_ref = hs2.hs2_sparse_attn_reuse(inp["q"], inp["k"], inp["v"], idx_t, cnt_t, **kw)
    o_na = torch.full_like(o_ref, 7)
    lse_na = torch.full_like(lse_ref, 7)
    hs2.hs2_sparse_attn_reuse_noalloc(inp["q"], inp["k"], inp["v"], idx_t, cnt_t, o=o_na, lse=lse_na, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o_na.view(torch.uint8), o_ref.view(torch.uint8))
    assert torch.equal(lse_na.view(torch.int32), lse_ref.view(torch.int32))
    return o_na, lse_na


def test_noalloc_matches_workspace_entry_point():
    say("noalloc: 48 queries x 9 pieces, bf16, H=16")
    inp, idx, cnt = _case(2, 24, 3000, 16, "bf16", 1152, 1)
    o, lse = _both(inp, idx, cnt)
    q64 = parity.decode(inp["q"])
    o_ref = np.zeros(q64.shape)
    for b in range(2):
        k64, v64 = parity.kv_f64(inp, b)
        for i in range(24):
            o_ref[b, i], _ = oracle.sparse_attn_reuse(q64[b, i], k64, v64, idx[b, i, : cnt[b, i]], 1 / 16)
    parity.check_out(o, o_ref, "bf16")

    say("noalloc: second call, smaller (7 queries x 5 pieces, e4m3, H=8)")
    _both(*_case(1, 7, 2000, 8, "e4m3", 600, 2))

    say("noalloc: the largest split size (64 queries x 16 pieces), f32, H=4")
    _both(*_case(4, 16, 2500, 4, "f32", 2048, 3))

    say("noalloc: one workgroup per query (80 queries, no scratch), bf16, H=2")
    _both(*_case(2, 40, 1500, 2, "bf16", 1152, 4))

    say("noalloc: a small call again after the largest")
    _both(*_case(1, 3, 900, 16, "bf16", 256, 5))


def test_noalloc_rejects_oversized_without_launching():
    inp, idx, cnt = _case(4, 16, 2500, 16, "bf16", 2176, 6)   # 64 x 17 slots > 1024
    with pytest.raises(hs2.Hs2Error) as e:
        hs2.hs2_sparse_attn_reuse_noalloc(inp["q"], inp["k"], inp["v"], torch.from_numpy(idx).to(DEV),
                                          torch.from_numpy(cnt).to(DEV), sm_scale=1 / 16)
    assert e.value.status == hs2.HS2_ERR_WORKSPACE

"""Every entry point run twice on the same inputs gives the same bytes.

The library promises deterministic results: there are no floating-point
atomics and no global-memory atomics (every partial result has its own slot,
and the multi-workgroup selector places each segment's candidates by a scan
of the segment counts); the selectors' LDS histograms count with integer
atomics, whose sums do not depend on the order.  Outputs are filled with
different bytes before each run, so an output element that a run does not
write also shows up as a difference.
"""
import numpy as np
import pytest
import torch

from token_level_sparse_full_amd import hs2, inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print("[case]", *a, flush=True)


def _twice(run, outs):
    """run(outs) writes into the tensors of outs; returns the two results as byte arrays."""
    res = []
    for fill in (0x00, 0xA5):
        for t in outs:
            t.view(torch.uint8).fill_(fill)
        run(outs)
        torch.cuda.synchronize()
        res.append([t.view(torch.uint8).cpu().numpy().copy() for t in outs])
    return res


def _same(res):
    for a, b in zip(*res):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("kv,H,n_q,T,q_pos0", [
    ("bf16", 16, 333, 700, 300),      # prefill, lse pass + P/V pass
    ("f32", 4, 200, 200, 0),          # prefill, f32 kernel
    ("e4m3", 16, 200, 500, 300),      # prefill, e4m3 kernel
    ("bf16", 16, 1, 40000, 39999),    # decode: split, merge tree, scores
    ("e4m3", 8, 2, 30000, 29998),
])
def test_full_attn_deterministic(kv, H, n_q, T, q_pos0):
    say("full", kv, H, n_q, T, q_pos0)
    B = 2
    inp = inputs.attention_inputs(B=B, n_q=n_q, T=T, H=H, d=256, kv=kv, n_sparse=0, seed=41, device=DEV)
    ld = (q_pos0 + n_q + 3) // 4 * 4
    o = torch.empty_like(inp["q"])
    lse = torch.empty((B, n_q, H), dtype=torch.float32, device=DEV)
    scores = torch.empty((B, n_q, ld), dtype=torch.float32, device=DEV)
    ws = hs2.workspace(hs2.full_attn_workspace_bytes(B, n_q, H, T, hs2._dtype_code(inp["k"])), DEV)

    def run(outs):
        scores.zero_()           # columns past each row's position are not written
        hs2.hs2_full_attn_scored(inp["q"], inp["k"], inp["v"], q_pos0=q_pos0, sm_scale=1 / 16,
                                 k_scale=inp["k_scale"], v_scale=inp["v_scale"], o=o, lse=lse, scores=scores,
                                 ld_scores=ld, ws=ws)
    _same(_twice(run, [o, lse]))
    a = scores.clone()
    run(None)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), scores.view(torch.int32))


@pytest.mark.parametrize("B,n_q,q_pos0", [(2, 300, 5000), (1, 2, 70000), (16, 1, 32767)])
def test_select_deterministic(B, n_q, q_pos0):
    say("select", B, n_q, q_pos0)
    g = torch.Generator(device=DEV)
    g.manual_seed(q_pos0)
    ld = (q_pos0 + n_q + 3) // 4 * 4
    sc = torch.rand((B, n_q, ld), generator=g, device=DEV)
    sc = torch.where(sc > 0.5, torch.round(sc * 64) / 64, sc * 1e-3)   # ties and spread
    idx = torch.empty((B, n_q, 1152), dtype=torch.int32, device=DEV)
    cnt = torch.empty((B, n_q), dtype=torch.int32, device=DEV)
    T = q_pos0 + n_q

    def run(outs):
        hs2.hs2_select_topk_window(sc, q_pos0=q_pos0, T=T, idx=idx, count=cnt)
    _same(_twice(run, [idx, cnt]))

    def run_b(outs):
        hs2.hs2_select_blocks_window(sc, q_pos0=q_pos0, T=T, block=64, idx=idx, count=cnt)
    _same(_twice(run_b, [idx, cnt]))


@pytest.mark.parametrize("kv,n_q", [("bf16", 24), ("bf16", 40), ("e4m3", 24), ("f32", 40)])
def test_sparse_deterministic(kv, n_q):
    say("sparse", kv, n_q)
    B, T, H = 2, 3000, 16
    inp = inputs.attention_inputs(B=B, n_q=n_q, T=T, H=H, d=256, kv=kv, n_sparse=0, seed=42, device=DEV)
    rng = np.random.default_rng(2)
    idx = np.full((B, n_q, 1152), -1, dtype=np.int32)
    cnt = np.zeros((B, n_q), dtype=np.int32)
    for b in range(B):
        for i in range(n_q):
            n = [0, 3, 129, 1152, 700][(b * n_q + i) % 5]
            idx[b, i, :n] = np.sort(rng.choice(T, size=n, replace=False))
            cnt[b, i] = n
    idx_t, cnt_t = torch.from_numpy(idx).to(DEV), torch.from_numpy(cnt).to(DEV)
    o = torch.empty_like(inp["q"])
    lse = torch.empty((B, n_q, H), dtype=torch.float32, device=DEV)

    def run(outs):
        hs2.hs2_sparse_attn_reuse(inp["q"], inp["k"], inp["v"], idx_t, cnt_t, sm_scale=1 / 16,
                                  k_scale=inp["k_scale"], v_scale=inp["v_scale"], o=o, lse=lse)
    _same(_twice(run, [o, lse]))


@pytest.mark.parametrize("fp8", [False, True])
def test_bridge_deterministic(fp8):
    say("bridge", fp8)
    L, D, nl = 700, 512, 2
    br = inputs.bridge_inputs(L=L, D=D, n_layers=nl, d=256, seed=43, device=DEV)
    if fp8:
        k = torch.empty((nl, L, 256), dtype=torch.uint8, device=DEV)
        v = torch.empty_like(k)
        ks = torch.empty((nl, L), dtype=torch.float32, device=DEV)
        vs = torch.empty_like(ks)
        outs = [k, v, ks, vs]

        def run(o):
            hs2.hs2_bridge_kv_proj_fp8(br["x"], br["w_k"], br["w_v"], k_out=k, v_out=v, k_scale=ks, v_scale=vs)
    else:
        k = torch.empty((nl, L, 256), dtype=torch.bfloat16, device=DEV)
        v = torch.empty_like(k)
        outs = [k, v]

        def run(o):
            hs2.hs2_bridge_kv_proj(br["x"], br["w_k"], br["w_v"], k_out=k, v_out=v)
    _same(_twice(run, outs))

"""The decode step as one unit: scored full attention, the selection and the
sparse layers captured into one HIP graph and replayed.

Every kernel of the step takes its scratch from caller-owned workspaces and
records no memset, so the step can be captured.  Each replay must reproduce
the eager step byte for byte; the outputs are cleared by eager work between
replays, so an output a replay does not write shows up as a difference.
"""
import pytest
import torch

from token_level_sparse_full_amd import hs2, inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"
SCALE = 1.0 / 16.0
MS = 128 + 1024


def say(*a):
    print("[case]", *a, flush=True)


def _step_buffers(q, qs, k, T, p):
    B, _, H, _ = q.shape
    ld = (p + 1 + 3) // 4 * 4
    return {
        "ws": hs2.workspace(hs2.full_attn_workspace_bytes(B, 1, H, T, hs2._dtype_code(k)), DEV),
        "ws_sel": hs2.workspace(hs2.select_workspace_bytes(B, 1, T, p), DEV),
        "ws_sp": hs2.workspace(hs2.sparse_workspace_bytes(B, 1, H, MS), DEV),
        "o": torch.empty_like(q), "lse": torch.empty((B, 1, H), dtype=torch.float32, device=DEV),
        "sc": torch.empty((B, 1, ld), dtype=torch.float32, device=DEV), "ld": ld,
        "idx": torch.empty((B, 1, MS), dtype=torch.int32, device=DEV),
        "cnt": torch.empty((B, 1), dtype=torch.int32, device=DEV),
        "o2": [torch.empty_like(x) for x in qs],
        "l2": [torch.empty((B, 1, H), dtype=torch.float32, device=DEV) for _ in qs],
    }


def _step(bf, q, qs, k, v, T, p, ks, vs):
    hs2.hs2_full_attn_scored(q, k, v, q_pos0=p, sm_scale=SCALE, k_scale=ks, v_scale=vs, o=bf["o"], lse=bf["lse"],
                             scores=bf["sc"], ld_scores=bf["ld"], ws=bf["ws"])
    hs2.hs2_select_topk_window(bf["sc"], q_pos0=p, T=T, idx=bf["idx"], count=bf["cnt"], ws=bf["ws_sel"])
    for i, x in enumerate(qs):
        hs2.hs2_sparse_attn_reuse(x, k, v, bf["idx"], bf["cnt"], sm_scale=SCALE, k_scale=ks, v_scale=vs,
                                  o=bf["o2"][i], lse=bf["l2"][i], ws=bf["ws_sp"])


def _outs(bf):
    return [bf["o"], bf["lse"], bf["sc"], bf["idx"], bf["cnt"], *bf["o2"], *bf["l2"]]


def _bits(t):
    return t.view(torch.uint8) if t.dtype != torch.int32 else t


# bf16: 4 sequences of 30000 keys (the multi-workgroup selector), 3 sparse layers;
# e4m3: one sequence of 70000 keys (a merge level above the chunk states), 4 sparse layers
@pytest.mark.parametrize("kv,B,T,n_sparse", [("bf16", 4, 30000, 3), ("e4m3", 1, 70000, 4)])
def test_decode_step_graph_replays(kv, B, T, n_sparse):
    say("decode graph", kv, B, T, n_sparse)
    inp = inputs.attention_inputs(B=B, n_q=1, T=T, H=16, d=256, kv=kv, n_sparse=n_sparse, seed=9, device=DEV)
    q, qs, k, v = inp["q"], inp["q_sparse"], inp["k"], inp["v"]
    ks, vs = inp["k_scale"], inp["v_scale"]
    p = T - 1
    bf = _step_buffers(q, qs, k, T, p)
    _step(bf, q, qs, k, v, T, p, ks, vs)
    torch.cuda.synchronize()
    ref = [x.clone() for x in _outs(bf)]

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(bf, q, qs, k, v, T, p, ks, vs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        _step(bf, q, qs, k, v, T, p, ks, vs)
    other = _step_buffers(q, qs, k, T, p)
    for rep in range(3):
        for x in _outs(bf):
            x.fill_(7)
        _step(other, q, qs, k, v, T, p, ks, vs)   # eager work of the program between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, _outs(bf)):
            assert torch.equal(_bits(a), _bits(b)), f"replay {rep} differs from the eager step"
    for a, b in zip(ref, _outs(other)):
        assert torch.equal(_bits(a), _bits(b))

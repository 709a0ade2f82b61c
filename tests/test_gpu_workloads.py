"""The five workloads at their own sizes, end to end through the C ABI, against
the float64 oracle.

Where the oracle can afford every output (tiny prefill, batched decode, the
1M-token FP8 decode steps, the bridge's attention steps) every output is
checked; for the 128k prefill and the bridge GEMM, sampled rows are checked one
by one and cheap invariants are checked on every row.  Each stage is checked
on the inputs the GPU stage consumed (the sparse layers on the GPU's own index
sets, the bridge's attention on the GPU-made K/V).  Rules: parity.py.
"""
import math
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
WIN, TOPK = 128, 1024


def say(*a):
    print("[case]", *a, flush=True)


def _check_select_rows(idx, cnt, s_gpu_rows, s_ref_rows, positions):
    """Exact on the GPU's own scores; within the tie band on the oracle's."""
    swaps = 0
    for r, p in enumerate(positions):
        parity.check_selection(idx[r], int(cnt[r]), s_gpu_rows[r][: p + 1].astype(np.float64), p, WIN, TOPK,
                               exact=True)
        swaps += parity.check_selection(idx[r], int(cnt[r]), s_ref_rows[r], p, WIN, TOPK)
    return swaps


def _sparse_layers(qs_list, k, v, idx, cnt, kind, k_scale=None, v_scale=None):
    return [hs2.hs2_sparse_attn_reuse(q, k, v, idx, cnt, sm_scale=1 / 16, k_scale=k_scale, v_scale=v_scale)
            for q in qs_list]


def test_tiny_prefill_2k():
    wl = inputs.WORKLOADS["tiny_prefill_2k"]
    say(wl.name)
    L, H = wl.L, wl.H
    inp = inputs.attention_inputs(B=1, n_q=L, T=L, H=H, d=256, kv="f32", n_sparse=1, seed=wl.seed, device=DEV)
    o, lse, scores = hs2.hs2_full_attn_scored(inp["q"], inp["k"], inp["v"], q_pos0=0, sm_scale=1 / 16)
    idx, cnt = hs2.hs2_select_topk_window(scores, q_pos0=0, T=L)
    (o2, lse2), = _sparse_layers(inp["q_sparse"], inp["k"], inp["v"], idx, cnt, "f32")
    torch.cuda.synchronize()
    k64, v64 = parity.kv_f64(inp, 0)
    q64 = parity.decode(inp["q"][0])
    o_ref, lse_ref, s_ref = oracle.full_attn_scored(q64, k64, v64, 0, 1 / 16)
    parity.check_out(o[0], o_ref, "f32")
    parity.check_lse(lse[0], lse_ref)
    s_np = scores[0].cpu().numpy()
    for i in range(L):
        parity.check_scores(s_np[i, : i + 1], s_ref[i], f"row {i}")
    idx_np, cnt_np = idx[0].cpu().numpy(), cnt[0].cpu().numpy()
    _check_select_rows(idx_np, cnt_np, s_np, s_ref, list(range(L)))
    q2 = parity.decode(inp["q_sparse"][0][0])
    o2_ref = np.stack([oracle.sparse_attn_reuse(q2[i], k64, v64, idx_np[i, : cnt_np[i]], 1 / 16)[0] for i in range(L)])
    parity.check_out(o2[0], o2_ref, "f32", "sparse o")


def test_decode_b16_32k():
    wl = inputs.WORKLOADS["decode_b16_32k"]
    say(wl.name)
    B, T, H = wl.B, wl.T, wl.H
    inp = inputs.attention_inputs(B=B, n_q=1, T=T, H=H, d=256, kv="bf16", n_sparse=wl.n_sparse, seed=wl.seed,
                                  device=DEV)
    o, lse, scores = hs2.hs2_full_attn_scored(inp["q"], inp["k"], inp["v"], q_pos0=T - 1, sm_scale=1 / 16)
    idx, cnt = hs2.hs2_select_topk_window(scores, q_pos0=T - 1, T=T)
    sp = _sparse_layers(inp["q_sparse"], inp["k"], inp["v"], idx, cnt, "bf16")
    torch.cuda.synchronize()
    s_np, idx_np, cnt_np = scores.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy()
    swaps = 0
    for b in range(B):
        k64, v64 = parity.kv_f64(inp, b)
        o_ref, lse_ref, s_ref = oracle.full_attn_scored(parity.decode(inp["q"][b]), k64, v64, T - 1, 1 / 16)
        parity.check_out(o[b], o_ref, "bf16")
        parity.check_lse(lse[b], lse_ref)
        parity.check_scores(s_np[b, 0, :T], s_ref[0], f"seq {b}")
        swaps += _check_select_rows(idx_np[b], cnt_np[b], s_np[b], s_ref, [T - 1])
        for layer, (o2, _) in enumerate(sp):
            q2 = parity.decode(inp["q_sparse"][layer][b, 0])
            o2_ref, _ = oracle.sparse_attn_reuse(q2, k64, v64, idx_np[b, 0, : cnt_np[b, 0]], 1 / 16)
            parity.check_out(o2[b, 0], o2_ref, "bf16", f"sparse layer {layer} seq {b}")
    print("boundary swaps within tolerance:", swaps)


def test_prefill_128k_sampled():
    wl = inputs.WORKLOADS["prefill_128k"]
    say(wl.name)
    L, H = wl.L, wl.H
    inp = inputs.attention_inputs(B=1, n_q=L, T=L, H=H, d=256, kv="bf16", n_sparse=wl.n_sparse, seed=wl.seed,
                                  device=DEV)
    needles = inputs.plant_needles(inp["q"][0], inp["k"][0], wl.needles, wl.seed)
    C = 32768
    idx = torch.empty((1, L, WIN + TOPK), dtype=torch.int32, device=DEV)
    cnt = torch.empty((1, L), dtype=torch.int32, device=DEV)
    o = torch.empty_like(inp["q"])
    lse = torch.empty((1, L, H), dtype=torch.float32, device=DEV)
    scores = torch.empty((1, C, L), dtype=torch.float32, device=DEV)
    rows = sorted({0, 1, 127, 128, 129, 1151, 1152, 1153, 4097, 32767, 32768, L // 2, L - 1} |
                  {i for _, i in needles[:12]})
    kept = {}
    # the block-level selection (ablation) of the same chunks, as bench.py launches it
    idx_b, cnt_b = torch.empty_like(idx), torch.empty_like(cnt)
    ws_b = hs2.workspace(hs2.select_blocks_workspace_bytes(1, C, L, L - C, WIN, 64), DEV)
    for c0 in range(0, L, C):
        hs2.hs2_full_attn_scored(inp["q"][:, c0:c0 + C], inp["k"], inp["v"], q_pos0=c0, sm_scale=1 / 16,
                                 o=o[:, c0:c0 + C], lse=lse[:, c0:c0 + C], scores=scores, ld_scores=L)
        for p in rows:
            if c0 <= p < c0 + C:
                kept[p] = scores[0, p - c0, : p + 1].cpu().numpy()
        hs2.hs2_select_topk_window(scores, q_pos0=c0, T=L, n_q=C, idx=idx[:, c0:c0 + C], count=cnt[:, c0:c0 + C])
        hs2.hs2_select_blocks_window(scores, q_pos0=c0, T=L, n_q=C, block=64, idx=idx_b[:, c0:c0 + C],
                                     count=cnt_b[:, c0:c0 + C], ws=ws_b)
    sp = _sparse_layers(inp["q_sparse"], inp["k"], inp["v"], idx, cnt, "bf16")
    torch.cuda.synchronize()
    # invariants on every row: count, window inside, strictly ascending, in range
    pos = torch.arange(L, device=DEV, dtype=torch.int32)
    assert torch.equal(cnt[0], torch.clamp(pos + 1, max=WIN + TOPK))
    full = cnt[0] == WIN + TOPK
    win = idx[0, full, TOPK:]
    assert torch.equal(win, (pos[full, None] - (WIN - 1) + torch.arange(WIN, device=DEV, dtype=torch.int32)))
    d = idx[0, full, 1:] - idx[0, full, :-1]
    assert (d > 0).all()
    # every needle is picked by its target query
    idx_np, cnt_np = idx[0].cpu().numpy(), cnt[0].cpu().numpy()
    # block-level selection of the sampled rows against the oracle's exact block sums on the GPU's scores
    idxb_np, cntb_np = idx_b[0].cpu().numpy(), cnt_b[0].cpu().numpy()
    for p in rows:
        parity.check_block_selection(idxb_np[p], int(cntb_np[p]), kept[p], p, WIN, TOPK, 64)
    for j, i in needles:
        assert j in idx_np[i, : cnt_np[i]], (j, i)
    # sampled rows against the oracle
    k64, v64 = parity.kv_f64(inp, 0)
    q_np = inputs.raw_numpy(inp["q"][0])
    o_np, lse_np = o[0].float().cpu().numpy(), lse[0].cpu().numpy()
    for p in rows:
        o_ref, lse_ref, s_ref = oracle.full_attn_scored(oracle.decode_rows(q_np[p:p + 1], "bf16"), k64, v64, p, 1 / 16)
        parity.check_out(torch.from_numpy(o_np[p]), o_ref[0], "bf16", f"o row {p}")
        parity.check_lse(torch.from_numpy(lse_np[p]), lse_ref[0])
        parity.check_scores(kept[p], s_ref[0], f"scores row {p}")
        _check_select_rows(idx_np[p:p + 1], cnt_np[p:p + 1], [kept[p]], s_ref, [p])
        for layer, (o2, _) in enumerate(sp):
            q2 = parity.decode(inp["q_sparse"][layer][0, p])
            o2_ref, _ = oracle.sparse_attn_reuse(q2, k64, v64, idx_np[p, : cnt_np[p]], 1 / 16)
            parity.check_out(o2[0, p], o2_ref, "bf16", f"sparse layer {layer} row {p}")


def test_bridge_64k():
    wl = inputs.WORKLOADS["bridge_64k"]
    say(wl.name)
    L, D, nl, H = wl.L, wl.D, wl.n_full, wl.H
    br = inputs.bridge_inputs(L=L, D=D, n_layers=nl, d=256, seed=wl.seed, device=DEV)
    k_all, v_all = hs2.hs2_bridge_kv_proj(br["x"], br["w_k"], br["w_v"])
    torch.cuda.synchronize()
    # sampled projection rows against float64 products (1 bf16 step + float32 accumulation bound)
    rng = np.random.default_rng(4)
    rows = np.sort(rng.choice(L, size=256, replace=False))
    x64 = parity.decode(br["x"][torch.from_numpy(rows).to(DEV)])
    wk64, wv64 = parity.decode(br["w_k"]), parity.decode(br["w_v"])
    k_ref, v_ref = oracle.bridge_kv_proj(x64, wk64, wv64)
    k_mag, v_mag = oracle.bridge_kv_proj(np.abs(x64), np.abs(wk64), np.abs(wv64))
    sel = torch.from_numpy(rows).to(DEV)
    for got_t, ref, mag in ((k_all[:, sel], k_ref, k_mag), (v_all[:, sel], v_ref, v_mag)):
        g = parity.decode(got_t.contiguous())
        ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
        assert (np.abs(g - ref) <= ulp + 64 * 2.0 ** -24 * mag).all()
    # each bridged full layer: one decode step at p = L-1 on the GPU-made cache,
    # selection, then the sparse layers that reuse it
    for m in range(nl):
        q = inputs.cast(inputs.normal((1, 1, H, 256), inputs.STD_QKV, wl.seed, inputs.S_QFULL_LAYER + m, DEV), "bf16")
        qs = [inputs.cast(inputs.normal((1, 1, H, 256), inputs.STD_QKV, wl.seed, inputs.S_QSPARSE + 8 * m + i, DEV),
                          "bf16") for i in range(wl.n_sparse)]
        k, v = k_all[m:m + 1], v_all[m:m + 1]
        o, lse, scores = hs2.hs2_full_attn_scored(q, k, v, q_pos0=L - 1, sm_scale=1 / 16)
        idx, cnt = hs2.hs2_select_topk_window(scores, q_pos0=L - 1, T=L)
        sp = _sparse_layers(qs, k, v, idx, cnt, "bf16")
        torch.cuda.synchronize()
        k64, v64 = parity.decode(k[0]), parity.decode(v[0])
        o_ref, lse_ref, s_ref = oracle.full_attn_scored(parity.decode(q[0]), k64, v64, L - 1, 1 / 16)
        parity.check_out(o[0], o_ref, "bf16")
        parity.check_lse(lse[0], lse_ref)
        s_np = scores[0].cpu().numpy()
        parity.check_scores(s_np[0, :L], s_ref[0], f"layer {m}")
        idx_np, cnt_np = idx[0].cpu().numpy(), cnt[0].cpu().numpy()
        _check_select_rows(idx_np, cnt_np, s_np, s_ref, [L - 1])
        for i, (o2, _) in enumerate(sp):
            o2_ref, _ = oracle.sparse_attn_reuse(parity.decode(qs[i][0, 0]), k64, v64, idx_np[0, : cnt_np[0]], 1 / 16)
            parity.check_out(o2[0, 0], o2_ref, "bf16", f"layer {m} sparse {i}")


def test_decode_1m_fp8():
    wl = inputs.WORKLOADS["decode_1m_fp8"]
    say(wl.name)
    T, H = wl.T, wl.H
    k, v, ks, vs = inputs.kv_cache((1, T, 256), "e4m3", wl.seed, DEV)
    k64 = oracle.decode_rows(inputs.raw_numpy(k[0]), "e4m3", inputs.raw_numpy(ks[0]))
    v64 = oracle.decode_rows(inputs.raw_numpy(v[0]), "e4m3", inputs.raw_numpy(vs[0]))
    for step in range(wl.steps):
        p = T - wl.steps + step
        say("step", step, "p", p)
        q = inputs.cast(inputs.normal((1, 1, H, 256), inputs.STD_QKV, wl.seed, inputs.S_Q + 10 * step, DEV), "bf16")
        qs = [inputs.cast(inputs.normal((1, 1, H, 256), inputs.STD_QKV, wl.seed, inputs.S_QSPARSE + 10 * step + i,
                                        DEV), "bf16") for i in range(wl.n_sparse)]
        o, lse, scores = hs2.hs2_full_attn_scored(q, k, v, q_pos0=p, sm_scale=1 / 16, k_scale=ks, v_scale=vs)
        idx, cnt = hs2.hs2_select_topk_window(scores, q_pos0=p, T=T)
        sp = _sparse_layers(qs, k, v, idx, cnt, "e4m3", ks, vs)
        torch.cuda.synchronize()
        o_ref, lse_ref, s_ref = oracle.full_attn_scored(parity.decode(q[0]), k64, v64, p, 1 / 16)
        parity.check_out(o[0], o_ref, "e4m3")
        parity.check_lse(lse[0], lse_ref)
        s_np = scores[0].cpu().numpy()
        parity.check_scores(s_np[0, : p + 1], s_ref[0], f"step {step}")
        idx_np, cnt_np = idx[0].cpu().numpy(), cnt[0].cpu().numpy()
        _check_select_rows(idx_np, cnt_np, s_np, s_ref, [p])
        for i, (o2, _) in enumerate(sp):
            o2_ref, _ = oracle.sparse_attn_reuse(parity.decode(qs[i][0, 0]), k64, v64, idx_np[0, : cnt_np[0]], 1 / 16)
            parity.check_out(o2[0, 0], o2_ref, "e4m3", f"step {step} sparse {i}")


def test_bridge_64k_fp8_every_position():
    """The bridge into the e4m3 cache at full size, then one bridged layer's
    cross-decoder at every prompt position (the many-query e4m3 path in the
    32768-query chunks bench.py times): sampled projection rows and sampled
    query rows of the last chunk against the oracle, the selection and a
    sparse layer of those rows on the GPU's own indices."""
    wl = inputs.WORKLOADS["bridge_64k"]
    say(wl.name, "fp8, every position")
    L, D, nl, H, C = wl.L, wl.D, wl.n_full, wl.H, 32768
    br = inputs.bridge_inputs(L=L, D=D, n_layers=nl, d=256, seed=wl.seed, device=DEV)
    k8, v8, ks, vs = hs2.hs2_bridge_kv_proj_fp8(br["x"], br["w_k"], br["w_v"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(44)
    rows = np.sort(np.concatenate([[0, L - 1], rng.choice(np.arange(1, L - 1), size=126, replace=False)]))
    x64 = parity.decode(br["x"][torch.from_numpy(rows).to(DEV)])
    wk64, wv64 = parity.decode(br["w_k"]), parity.decode(br["w_v"])
    kc_r, vc_r, ks_r, vs_r = oracle.bridge_kv_proj_fp8(x64, wk64, wv64)
    k_ref, v_ref = oracle.bridge_kv_proj(x64, wk64, wv64)
    k_abs, v_abs = oracle.bridge_kv_proj(np.abs(x64), np.abs(wk64), np.abs(wv64))
    table = oracle.e4m3_decode_table()
    sel_rows = torch.from_numpy(rows).to(DEV)
    for codes, sc, ref, mag, codes_r, sc_r in ((k8, ks, k_ref, k_abs, kc_r, ks_r), (v8, vs, v_ref, v_abs, vc_r, vs_r)):
        c = codes[:, sel_rows].cpu().numpy()
        s_ = sc[:, sel_rows].cpu().numpy().astype(np.float64)
        slack = 64 * 2.0 ** -24 * mag
        assert (np.abs(s_ - sc_r) <= slack.max(axis=-1) / 448.0 + 2.0 ** -23 * sc_r).all()
        got = table[c] * s_[..., None]
        step = np.maximum(2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref) / s_[..., None], 2.0 ** -6))) - 3),
                          2.0 ** -9) * s_[..., None]
        assert (np.abs(got - ref) <= 1.5 * step + 2 * slack).all()
        assert (c == codes_r).mean() > 0.999
    # layer 0 on its e4m3 cache: the last query chunk, as bench.py launches it
    m, c0 = 0, L - C
    q = inputs.cast(inputs.normal((1, L, H, 256), inputs.STD_QKV, wl.seed, inputs.S_QFULL_LAYER + m, DEV), "bf16")
    q2 = inputs.cast(inputs.normal((1, L, H, 256), inputs.STD_QKV, wl.seed, inputs.S_QSPARSE + 8 * m, DEV), "bf16")
    k, v, ksm, vsm = k8[m:m + 1], v8[m:m + 1], ks[m:m + 1], vs[m:m + 1]
    o, lse, scores = hs2.hs2_full_attn_scored(q[:, c0:], k, v, q_pos0=c0, sm_scale=1 / 16, k_scale=ksm, v_scale=vsm,
                                              ld_scores=L)
    idx, cnt = hs2.hs2_select_topk_window(scores, q_pos0=c0, T=L)
    o2, _ = hs2.hs2_sparse_attn_reuse(q2[:, c0:], k, v, idx, cnt, sm_scale=1 / 16, k_scale=ksm, v_scale=vsm)
    torch.cuda.synchronize()
    k64 = oracle.decode_rows(inputs.raw_numpy(k[0]), "e4m3", inputs.raw_numpy(ksm[0]))
    v64 = oracle.decode_rows(inputs.raw_numpy(v[0]), "e4m3", inputs.raw_numpy(vsm[0]))
    qi = np.sort(np.concatenate([[0, C - 1], rng.choice(np.arange(1, C - 1), size=4, replace=False)]))
    qsel = torch.from_numpy(qi).to(DEV)
    q64 = parity.decode(q[0, c0:][qsel])
    q264 = parity.decode(q2[0, c0:][qsel])
    s_rows = scores[0, qsel].cpu().numpy()
    idx_np, cnt_np = idx[0, qsel].cpu().numpy(), cnt[0, qsel].cpu().numpy()
    s_refs = []
    for r, i in enumerate(qi):
        p = c0 + int(i)
        say("query row", p)
        o_ref, lse_ref, s_ref = oracle.full_attn_scored(q64[r:r + 1], k64, v64, p, 1 / 16)
        parity.check_out(o[0, int(i):int(i) + 1], o_ref, "e4m3", f"o row {p}")
        parity.check_lse(lse[0, int(i):int(i) + 1], lse_ref)
        parity.check_scores(s_rows[r, : p + 1], s_ref[0], f"scores row {p}")
        s_refs.append(s_ref[0])
        o2_ref, _ = oracle.sparse_attn_reuse(q264[r], k64, v64, idx_np[r, : cnt_np[r]], 1 / 16)
        parity.check_out(o2[0, int(i)], o2_ref, "e4m3", f"sparse row {p}")
    _check_select_rows(idx_np, cnt_np, s_rows, s_refs, [c0 + int(i) for i in qi])


def test_self_decoder_swa_128k_sampled():
    """The self-decoder's SWA layer over the 128k prompt (window 128, 64-dim
    partial RoPE, base 10000), as bench.py launches it (the rotary embedding of
    Q and K, then the attention): sampled query rows (the sequence start, the
    window edge, the middle and the end) against the oracle."""
    wl = inputs.WORKLOADS["self_decoder_swa_128k"]
    say(wl.name)
    L, H = wl.L, wl.H
    inp = inputs.attention_inputs(B=1, n_q=L, T=L, H=H, d=256, kv="bf16", n_sparse=0, seed=wl.seed, device=DEV)
    qr = hs2.hs2_rope_partial(inp["q"][0], pos0=0, rope_dims=wl.rope_dims, rope_base=10000.0)[None]
    kr = hs2.hs2_rope_partial(inp["k"][0], pos0=0, rope_dims=wl.rope_dims, rope_base=10000.0)[None]
    o, lse = hs2.hs2_swa_attn(qr, kr, inp["v"], q_pos0=0, window=wl.window, sm_scale=1 / 16)
    torch.cuda.synchronize()
    rng = np.random.default_rng(6)
    rows = sorted({0, 1, 126, 127, 128, 129, 4095, L // 2, L - 2, L - 1} | set(rng.integers(0, L, 22).tolist()))
    for p in rows:
        lo = max(0, p - wl.window + 1)
        k64 = np.zeros((p + 1, 256))
        v64 = np.zeros((p + 1, 256))
        k64[lo:] = parity.decode(inp["k"][0, lo: p + 1])
        v64[lo:] = parity.decode(inp["v"][0, lo: p + 1])
        o_ref, lse_ref = oracle.swa_attn(parity.decode(inp["q"][0, p: p + 1]), k64, v64, p, wl.window, wl.rope_dims,
                                         10000.0, 1 / 16)
        parity.check_out(o[0, p: p + 1], o_ref, "bf16", f"o row {p}")
        parity.check_lse(lse[0, p: p + 1], lse_ref)

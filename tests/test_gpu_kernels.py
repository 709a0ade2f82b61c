"""GPU parity of each C-ABI entry point against the float64 oracle.

Sizes are small enough for the oracle to finish in seconds while spanning
several key tiles, several workgroups and ragged tails.  The acceptance rules
are stated in parity.py.
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
SCALE = 1.0 / 16.0


def say(*a):
    print("[case]", *a, flush=True)


# --------------------------------------------------------------------------- sparse reuse
def _random_sets(rng, B, n_q, T, sizes, max_sel, with_invalid):
    idx = np.full((B, n_q, max_sel), -1, dtype=np.int32)
    cnt = np.zeros((B, n_q), dtype=np.int32)
    for b in range(B):
        for i in range(n_q):
            n = sizes[(b * n_q + i) % len(sizes)]
            sel = rng.choice(T, size=n, replace=False).astype(np.int32)
            if with_invalid and n > 3 and i % 3 == 0:
                sel[rng.integers(0, n)] = -1
                sel[rng.integers(0, n)] = T + int(rng.integers(0, 5))
            idx[b, i, :n] = sel
            cnt[b, i] = n
    return idx, cnt


# Every (cache dtype, H) instance in both forms: B * n_q = 48 takes the split form (128-key
# pieces merged by a second kernel), 80 one workgroup per query.
@pytest.mark.parametrize("kv,H,n_q", [(kv, H, n_q) for kv in ("bf16", "e4m3", "f32") for H in (1, 2, 4, 8, 16)
                                      for n_q in (24, 40)])
def test_sparse_reuse_parity(kv, H, n_q):
    say("sparse", kv, H, n_q)
    B, T, max_sel = 2, 3000, 1152
    inp = inputs.attention_inputs(B=B, n_q=n_q, T=T, H=H, d=256, kv=kv, n_sparse=0, seed=11, device=DEV)
    rng = np.random.default_rng(5)
    idx, cnt = _random_sets(rng, B, n_q, T, [0, 1, 5, 31, 32, 33, 100, 1152, 700, 17], max_sel, True)
    o, lse = hs2.hs2_sparse_attn_reuse(inp["q"], inp["k"], inp["v"], torch.from_numpy(idx).to(DEV),
                                       torch.from_numpy(cnt).to(DEV), sm_scale=SCALE,
                                       k_scale=inp["k_scale"], v_scale=inp["v_scale"])
    torch.cuda.synchronize()
    q64 = parity.decode(inp["q"])
    o_ref = np.zeros((B, n_q, H, 256))
    lse_ref = np.zeros((B, n_q, H))
    for b in range(B):
        k64, v64 = parity.kv_f64(inp, b)
        for i in range(n_q):
            sel = idx[b, i, : cnt[b, i]]
            sel = sel[(sel >= 0) & (sel < T)]
            o_ref[b, i], lse_ref[b, i] = oracle.sparse_attn_reuse(q64[b, i], k64, v64, sel, SCALE)
    parity.check_out(o, o_ref, kv)
    lg = lse.cpu().numpy()
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lg), empty)
    parity.check_lse(torch.from_numpy(lg[~empty]), lse_ref[~empty])


# --------------------------------------------------------------------------- selection
def _select_case(scores_np, q_pos0, T, window, topk):
    B, n_q, ld = scores_np.shape
    s = torch.from_numpy(scores_np).to(DEV)
    idx, cnt = hs2.hs2_select_topk_window(s, q_pos0=q_pos0, T=T, window=window, topk=topk)
    torch.cuda.synchronize()
    idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    for b in range(B):
        for i in range(n_q):
            p = q_pos0 + i
            parity.check_selection(idx[b, i], int(cnt[b, i]), scores_np[b, i, : p + 1].astype(np.float64), p,
                                   window, topk, exact=True)


@pytest.mark.parametrize("q_pos0,n_q,T", [(0, 140, 200), (1100, 200, 1400), (9000, 40, 9100), (40000, 3, 40004)])
def test_select_parity(q_pos0, n_q, T):
    say("select", q_pos0, n_q, T)
    rng = np.random.default_rng(q_pos0 + 7)
    ld = (q_pos0 + n_q + 3) // 4 * 4
    B = 2
    sc = np.zeros((B, n_q, ld), dtype=np.float32)
    for b in range(B):
        for i in range(n_q):
            n = q_pos0 + i + 1
            mode = (b * n_q + i) % 6
            if mode == 0:      # smooth random
                row = rng.random(n, dtype=np.float32) / n
            elif mode == 1:    # heavy ties
                row = (rng.integers(0, 7, n) / 64.0).astype(np.float32)
            elif mode == 2:    # all equal
                row = np.full(n, 1.0 / n, dtype=np.float32)
            elif mode == 3:    # zeros with a few spikes
                row = np.zeros(n, dtype=np.float32)
                row[rng.integers(0, n, size=min(n, 50))] = 1.0
            elif mode == 4:    # near-uniform: differences only in low mantissa bits
                row = (np.float32(1.0 / 4096) * (1 + rng.integers(0, 16, n) * np.float32(2 ** -20))).astype(np.float32)
            else:              # spread over many octaves
                row = (rng.lognormal(0.0, 3.0, n) / n).astype(np.float32)
            sc[b, i, :n] = row
    _select_case(sc, q_pos0, T, 128, 1024)


# Rows with a sink (a few candidates scoring 2.0 or more, as scores summed over heads can)
# next to heavy ties and 1-ulp neighbours at the cut: the exact threshold then spans 31 bits
# of the float32 pattern.  Short rows (kept whole in LDS), sampled long rows, and few long
# rows (the multi-workgroup form).
@pytest.mark.parametrize("q_pos0,n_q,T", [(2900, 24, 3000), (9000, 16, 9100), (40000, 3, 40004)])
def test_select_sink_and_ties(q_pos0, n_q, T):
    say("select sink", q_pos0, n_q, T)
    rng = np.random.default_rng(q_pos0 + 3)
    ld = (q_pos0 + n_q + 3) // 4 * 4
    B = 2
    sc = np.zeros((B, n_q, ld), dtype=np.float32)
    base = np.float32(1e-3)
    ulp = np.spacing(base)
    for b in range(B):
        for i in range(n_q):
            n = q_pos0 + i + 1
            row = base + ulp * rng.integers(-2, 3, n).astype(np.float32)
            row[rng.integers(0, n, size=600)] = base * np.float32(1.5)
            row[rng.integers(0, n - 128, size=1 + (b * n_q + i) % 3)] = np.float32(3.0 + i % 2)
            if i % 4 == 1:
                row[rng.integers(0, n - 128, size=2)] = np.float32(2.0)
            sc[b, i, :n] = row.astype(np.float32)
    _select_case(sc, q_pos0, T, 128, 1024)


# Few long rows (the multi-workgroup form, from 24576 candidates on): each segment of 4096
# candidates stores at most 512 of those at or above the row's threshold estimate, so rows
# whose best candidates crowd into one or two segments take the path that reads such a
# segment again; a row that keeps too few or too many over the estimate takes the exact
# multi-pass path.  Just above the size where the form starts, and at 70k.
@pytest.mark.parametrize("q_pos0,n_q,T", [(24720, 2, 24730), (70000, 1, 70001)])
def test_select_few_rows_crowded(q_pos0, n_q, T):
    say("select crowded", q_pos0, n_q, T)
    rng = np.random.default_rng(q_pos0 + 11)
    ld = (q_pos0 + n_q + 3) // 4 * 4
    B = 5
    sc = np.zeros((B, n_q, ld), dtype=np.float32)
    for b in range(B):
        for i in range(n_q):
            n = q_pos0 + i + 1
            nc = n - 128
            row = rng.random(n, dtype=np.float32) / n
            mode = (b * n_q + i) % 5
            if mode == 0:      # 2000 strong candidates inside one segment
                row[8192 + rng.choice(4096, size=2000, replace=False)] += np.float32(8.0 / n)
            elif mode == 1:    # a strong run across a segment boundary, with ties in it
                row[3000:7500] = np.float32(4.0 / n) + np.float32(1.0 / n) * rng.integers(0, 4, 4500)
            elif mode == 2:    # decreasing: the best candidates are the first ones
                row[:nc] = (np.arange(nc, 0, -1, dtype=np.float64) / (float(n) * n)).astype(np.float32)
            elif mode == 3:    # a crowded segment at the end of the candidates
                row[nc - 3000:nc] += np.float32(2.0 / n)
            else:              # heavy ties everywhere: the estimate keeps too many
                row = (rng.integers(0, 3, n) / 64.0).astype(np.float32)
            sc[b, i, :n] = row
    _select_case(sc, q_pos0, T, 128, 1024)


def _score_rows(rng, B, n_q, q_pos0, ld):
    sc = np.zeros((B, n_q, ld), dtype=np.float32)
    for b in range(B):
        for i in range(n_q):
            n = q_pos0 + i + 1
            mode = (b * n_q + i) % 5
            if mode == 0:      # smooth random
                row = rng.random(n, dtype=np.float32) / n
            elif mode == 1:    # heavy ties (many equal block sums)
                row = (rng.integers(0, 3, n) / 64.0).astype(np.float32)
            elif mode == 2:    # all equal
                row = np.full(n, 1.0 / n, dtype=np.float32)
            elif mode == 3:    # zeros with a few spikes
                row = np.zeros(n, dtype=np.float32)
                row[rng.integers(0, n, size=min(n, 50))] = 1.0
            else:              # spread over many octaves: the summation order shows in the sums
                row = (rng.lognormal(0.0, 3.0, n) / n).astype(np.float32)
            sc[b, i, :n] = row
    return sc


# block-level selection against the oracle's exact block sums, within the band that the
# kernel's float32 pairwise-tree sums allow (parity.check_block_selection).  Cases: rows below
# and above the cut, partial last blocks, 2.5k and 9.4k candidate blocks (both LDS
# capacities), blocks of 4..256.
@pytest.mark.parametrize("q_pos0,n_q,window,topk,block", [
    (1100, 200, 128, 1024, 64),
    (9000, 40, 128, 1024, 64),
    (40000, 3, 128, 1024, 16),
    (300000, 2, 128, 1024, 32),
    (5000, 9, 128, 1024, 256),
    (0, 70, 2, 8, 4),
    (700, 33, 5, 24, 8),
    (2000, 17, 128, 512, 128),
])
def test_select_blocks_parity(q_pos0, n_q, window, topk, block):
    say("select blocks", q_pos0, n_q, window, topk, block)
    rng = np.random.default_rng(q_pos0 + block)
    ld = (q_pos0 + n_q + 3) // 4 * 4
    B = 2
    sc = _score_rows(rng, B, n_q, q_pos0, ld)
    T = q_pos0 + n_q
    idx, cnt = hs2.hs2_select_blocks_window(torch.from_numpy(sc).to(DEV), q_pos0=q_pos0, T=T, window=window,
                                            topk=topk, block=block)
    torch.cuda.synchronize()
    idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    swaps = 0
    for b in range(B):
        for i in range(n_q):
            p = q_pos0 + i
            swaps += parity.check_block_selection(idx[b, i], int(cnt[b, i]), sc[b, i], p, window, topk, block)
    print("block swaps within the band:", swaps)


def test_select_blocks_feeds_sparse_layer():
    """The block selection of the GPU's own scores drives the sparse layer unchanged."""
    say("select blocks -> sparse")
    inp = inputs.attention_inputs(B=1, n_q=64, T=1600, H=16, d=256, kv="bf16", n_sparse=1, seed=12, device=DEV)
    q_pos0 = 1536
    _, _, scores = hs2.hs2_full_attn_scored(inp["q"], inp["k"], inp["v"], q_pos0=q_pos0, sm_scale=SCALE)
    idx, cnt = hs2.hs2_select_blocks_window(scores, q_pos0=q_pos0, T=1600, block=64)
    o, lse = hs2.hs2_sparse_attn_reuse(inp["q_sparse"][0], inp["k"], inp["v"], idx, cnt, sm_scale=SCALE)
    torch.cuda.synchronize()
    s_np, idx_np, cnt_np = scores.cpu().numpy()[0], idx.cpu().numpy()[0], cnt.cpu().numpy()[0]
    k64, v64 = parity.kv_f64(inp, 0)
    q64 = parity.decode(inp["q_sparse"][0][0])
    o_ref = np.zeros_like(q64)
    lse_ref = np.zeros(q64.shape[:2])
    for i in range(64):
        p = q_pos0 + i
        parity.check_block_selection(idx_np[i], int(cnt_np[i]), s_np[i], p, 128, 1024, 64)
        o_ref[i], lse_ref[i] = oracle.sparse_attn_reuse(q64[i], k64, v64, idx_np[i, : cnt_np[i]], SCALE)
    parity.check_out(o[0], o_ref, "bf16")
    parity.check_lse(lse[0], lse_ref)


def test_select_small_window_topk():
    say("select small")
    rng = np.random.default_rng(3)
    q_pos0, n_q, T = 0, 64, 64
    sc = (rng.integers(0, 5, size=(1, n_q, 64)) / 8.0).astype(np.float32)
    _select_case(sc, q_pos0, T, 2, 3)


# --------------------------------------------------------------------------- scored full attention
def _oracle_full(inp, b, q_pos0):
    k64, v64 = parity.kv_f64(inp, b)
    q64 = parity.decode(inp["q"][b])
    return oracle.full_attn_scored(q64, k64, v64, q_pos0, SCALE)


def _check_full(inp, o, lse, scores, q_pos0, kv, large_logits=False):
    B, n_q = inp["q"].shape[:2]
    s_np = scores.cpu().numpy()
    for b in range(B):
        o_ref, lse_ref, s_ref = _oracle_full(inp, b, q_pos0)
        parity.check_out(o[b], o_ref, kv)
        parity.check_lse(lse[b], lse_ref)
        # the score bound grows with the logits' magnitude (the largest logit of a row is
        # within ln(p + 1) of its lse)
        rel = parity.scores_rel_for_logits(np.abs(lse_ref).max() / math.log(2.0)) if large_logits else parity.S_REL
        for i in range(n_q):
            p = q_pos0 + i
            parity.check_scores(s_np[b, i, : p + 1], s_ref[i], f"scores b={b} i={i}", rel)


@pytest.mark.parametrize("kv,H,q_pos0,n_q,T", [
    ("bf16", 16, 300, 333, 700),
    ("bf16", 16, 0, 70, 70),
    ("bf16", 8, 130, 77, 300),
    ("bf16", 4, 5, 100, 110),
    ("f32", 4, 0, 200, 200),
    ("f32", 16, 64, 40, 104),
    ("bf16", 2, 0, 50, 50),
    ("bf16", 1, 10, 90, 100),
    ("e4m3", 16, 300, 333, 700),
    ("e4m3", 16, 0, 70, 70),
    ("e4m3", 8, 130, 77, 300),
    ("e4m3", 4, 5, 100, 110),
    ("e4m3", 1, 10, 90, 100),
    ("e4m3", 2, 33, 60, 93),
    ("f32", 1, 0, 150, 150),
    ("f32", 2, 20, 90, 110),
    ("f32", 8, 100, 70, 170),
])
def test_full_attn_prefill_parity(kv, H, q_pos0, n_q, T):
    say("prefill", kv, H, q_pos0, n_q, T)
    inp = inputs.attention_inputs(B=2, n_q=n_q, T=T, H=H, d=256, kv=kv, n_sparse=0, seed=21, device=DEV)
    o, lse, scores = hs2.hs2_full_attn_scored(inp["q"], inp["k"], inp["v"], q_pos0=q_pos0, sm_scale=SCALE,
                                              k_scale=inp["k_scale"], v_scale=inp["v_scale"])
    torch.cuda.synchronize()
    _check_full(inp, o, lse, scores, q_pos0, kv)


# Logits that jump far above everything before them partway along the row (a key block
# aligned with the queries): the lse pass of the bf16 and e4m3 caches keeps a lazy reference
# maximum and must redo such tiles against the true one.  Keys 500.. and 900.. raise the
# logits by about 104 and then 69 (log2 units), more than the 60 the lazy reference
# tolerates; queries 400..1099 see neither, the first, or both jumps.
@pytest.mark.parametrize("kv", ["bf16", "e4m3"])
def test_full_attn_prefill_logit_jump(kv):
    say("prefill logit jump", kv)
    B, H, q_pos0, n_q, T = 2, 16, 400, 700, 1100
    qk = inputs.q_dtype_of(kv)
    qf = inputs.normal((B, n_q, H, 256), inputs.STD_QKV, 41, inputs.S_Q, DEV)
    qf[..., 0] += 1.0
    kf = inputs.normal((B, T, 256), inputs.STD_QKV, 41, inputs.S_K, DEV)
    kf[:, 500:, 0] = 1152.0
    kf[:, 900:, 0] = 1920.0
    vf = inputs.normal((B, T, 256), inputs.STD_QKV, 41, inputs.S_V, DEV)
    if kv == "e4m3":
        k, ks = inputs.quantize_e4m3_rows(kf)
        v, vs = inputs.quantize_e4m3_rows(vf)
    else:
        k, v, ks, vs = inputs.cast(kf, kv), inputs.cast(vf, kv), None, None
    inp = dict(q=inputs.cast(qf, qk), k=k, v=v, k_scale=ks, v_scale=vs, kv=kv, q_kind=qk)
    o, lse, scores = hs2.hs2_full_attn_scored(inp["q"], k, v, q_pos0=q_pos0, sm_scale=SCALE, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    _check_full(inp, o, lse, scores, q_pos0, kv, large_logits=True)


@pytest.mark.parametrize("kv,H,n_q,T,q_pos0", [
    ("bf16", 16, 1, 5000, 4999),
    ("bf16", 16, 1, 5000, 3000),
    ("e4m3", 16, 1, 5000, 4999),
    ("f32", 16, 1, 700, 699),
    ("bf16", 8, 2, 2100, 2098),
    ("bf16", 4, 4, 300, 200),
    ("e4m3", 4, 2, 3000, 2998),
    ("bf16", 1, 16, 2000, 1984),
    ("bf16", 1, 5, 900, 800),
    ("bf16", 2, 8, 1500, 1492),
    ("bf16", 2, 3, 600, 597),
    ("e4m3", 1, 16, 2500, 2484),
    ("e4m3", 2, 8, 1200, 1000),
    ("e4m3", 8, 2, 4100, 4098),
    ("f32", 1, 16, 700, 684),
    ("f32", 2, 8, 800, 792),
    ("f32", 4, 4, 640, 636),
    ("f32", 8, 2, 900, 898),
])
def test_full_attn_decode_parity(kv, H, n_q, T, q_pos0):
    say("decode", kv, H, n_q, T, q_pos0)
    inp = inputs.attention_inputs(B=3, n_q=n_q, T=T, H=H, d=256, kv=kv, n_sparse=0, seed=31, device=DEV)
    o, lse, scores = hs2.hs2_full_attn_scored(inp["q"], inp["k"], inp["v"], q_pos0=q_pos0, sm_scale=SCALE,
                                              k_scale=inp["k_scale"], v_scale=inp["v_scale"])
    torch.cuda.synchronize()
    _check_full(inp, o, lse, scores, q_pos0, kv)


def test_full_attn_leaves_other_columns_untouched():
    say("untouched columns")
    inp = inputs.attention_inputs(B=1, n_q=20, T=64, H=16, d=256, kv="bf16", n_sparse=0, seed=3, device=DEV)
    scores = torch.full((1, 20, 64), -7.0, device=DEV)
    hs2.hs2_full_attn_scored(inp["q"], inp["k"], inp["v"], q_pos0=40, sm_scale=SCALE, scores=scores, ld_scores=64)
    torch.cuda.synchronize()
    s = scores.cpu().numpy()[0]
    for i in range(20):
        assert (s[i, 41 + i:] == -7.0).all()
        assert (s[i, : 41 + i] >= 0).all()


# --------------------------------------------------------------------------- bridge
def _bf16_from_f32(x):
    return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)


# D / 32 chunks of the K dimension: 1, 3, 5, 7 exercise the pipeline's partial rounds of 4 stage
# buffers and the chunks past the end; L not a multiple of 256 the rows past L
# 9000 rows x 4 layers are 288 tiles of 256 x 256, more than one round of workgroups.
# D / 32 chunks of K: the main loop takes groups of four, the tail the other 1, 2 or 3.
@pytest.mark.parametrize("L,D,n_layers", [(300, 256, 2), (1, 2048, 4), (513, 512, 1), (257, 32, 1), (100, 96, 3),
                                          (70, 160, 2), (513, 224, 1), (130, 192, 2), (40, 64, 1), (9000, 256, 4),
                                          (9000, 160, 4)])
def test_bridge_integer_exact(L, D, n_layers):
    say("bridge int", L, D, n_layers)
    rng = np.random.default_rng(L + D)
    x = rng.integers(-8, 9, size=(L, D))
    wk = rng.integers(-4, 5, size=(n_layers, D, 256))
    wv = rng.integers(-4, 5, size=(n_layers, D, 256))
    k, v = hs2.hs2_bridge_kv_proj(_bf16_from_f32(x).to(DEV), _bf16_from_f32(wk).to(DEV), _bf16_from_f32(wv).to(DEV))
    torch.cuda.synchronize()
    k_ref, v_ref = oracle.bridge_kv_proj(x.astype(np.float64), wk.astype(np.float64), wv.astype(np.float64))
    assert np.array_equal(inputs.raw_numpy(k), oracle.f64_to_bf16_bits(k_ref))
    assert np.array_equal(inputs.raw_numpy(v), oracle.f64_to_bf16_bits(v_ref))


def test_bridge_normal_within_one_ulp_and_strided_output():
    say("bridge normal")
    L, D, n_layers, T = 700, 2048, 2, 1024
    inp = inputs.bridge_inputs(L=L, D=D, n_layers=n_layers, d=256, seed=4, device=DEV)
    k_cache = torch.zeros((n_layers, T, 256), dtype=torch.bfloat16, device=DEV)
    v_cache = torch.zeros((n_layers, T, 256), dtype=torch.bfloat16, device=DEV)
    hs2.hs2_bridge_kv_proj(inp["x"], inp["w_k"], inp["w_v"], k_out=k_cache, v_out=v_cache, out_layer_stride=T * 256)
    torch.cuda.synchronize()
    x64, wk64, wv64 = parity.decode(inp["x"]), parity.decode(inp["w_k"]), parity.decode(inp["w_v"])
    k_ref, v_ref = oracle.bridge_kv_proj(x64, wk64, wv64)
    # |sum| of |x w| bounds the float32 accumulation error: allow 64 roundings of
    # 2**-24 on that scale, plus one bf16 step of the result (the float32 sum may
    # sit on the other side of a rounding boundary).
    k_abs, v_abs = oracle.bridge_kv_proj(np.abs(x64), np.abs(wk64), np.abs(wv64))
    for got, ref, mag in ((k_cache[:, :L], k_ref, k_abs), (v_cache[:, :L], v_ref, v_abs)):
        g = parity.decode(got.contiguous())
        ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
        assert (np.abs(g - ref) <= ulp + 64 * 2.0 ** -24 * mag).all()
        assert (np.abs(g - ref) <= ulp).mean() > 0.999
    assert (k_cache[:, L:] == 0).all() and (v_cache[:, L:] == 0).all()

# --------------------------------------------------------------------------- bridge into an e4m3 cache
@pytest.mark.parametrize("L,D,n_layers", [(300, 256, 2), (70, 160, 1), (1, 2048, 4), (130, 192, 1), (97, 96, 2),
                                          (40, 64, 1), (9000, 256, 4), (9000, 160, 4)])
def test_bridge_fp8_integer_exact(L, D, n_layers):
    """Integer inputs make the float32 accumulators exact, so codes and scales
    must equal the oracle's bit for bit (row 0 is all zero: scale 1, codes 0)."""
    say("bridge fp8 int", L, D, n_layers)
    rng = np.random.default_rng(L + 3 * D)
    x = rng.integers(-8, 9, size=(L, D))
    x[0] = 0
    wk = rng.integers(-4, 5, size=(n_layers, D, 256))
    wv = rng.integers(-4, 5, size=(n_layers, D, 256))
    kc, vc, ks, vs = hs2.hs2_bridge_kv_proj_fp8(_bf16_from_f32(x).to(DEV), _bf16_from_f32(wk).to(DEV),
                                               _bf16_from_f32(wv).to(DEV))
    torch.cuda.synchronize()
    kc_r, vc_r, ks_r, vs_r = oracle.bridge_kv_proj_fp8(x.astype(np.float64), wk.astype(np.float64),
                                                       wv.astype(np.float64))
    np.testing.assert_array_equal(ks.cpu().numpy(), ks_r)
    np.testing.assert_array_equal(vs.cpu().numpy(), vs_r)
    np.testing.assert_array_equal(kc.cpu().numpy(), kc_r)
    np.testing.assert_array_equal(vc.cpu().numpy(), vc_r)


def test_bridge_fp8_quotient_ties():
    """Rows whose quotients v / scale fall exactly on, or one float32 step off, an e4m3
    tie: the codes must be those of the IEEE float32 quotient (not of the product
    with the reciprocal of the scale, which lands on the other side of the tie)."""
    say("bridge fp8 ties")
    # every value is exact in bf16 (at most 8 significant bits)
    pairs = [(52, 39), (104, 39), (104, 78), (124, 93), (196, 175), (204, 153), (208, 39), (248, 93),
             (248, 186), (392, 175), (392, 203), (392, 350)]
    D, L = 32, len(pairs) * 2
    x = np.zeros((L, D))
    wk = np.zeros((1, D, 256))
    wv = np.zeros((1, D, 256))
    for r, (amax, a) in enumerate(pairs):
        x[2 * r, r] = 1.0          # row 2r: +amax, +a, -a spread over the columns
        x[2 * r + 1, r] = -1.0     # row 2r+1: the negated row
        wk[0, r, :3] = [amax, a, -a]
        wv[0, r, 5:7] = [a, amax]
    xb, wkb, wvb = _bf16_from_f32(x), _bf16_from_f32(wk), _bf16_from_f32(wv)
    kc, vc, ks, vs = hs2.hs2_bridge_kv_proj_fp8(xb.to(DEV), wkb.to(DEV), wvb.to(DEV))
    torch.cuda.synchronize()
    kc_r, vc_r, ks_r, vs_r = oracle.bridge_kv_proj_fp8(parity.decode(xb), parity.decode(wkb), parity.decode(wvb))
    np.testing.assert_array_equal(ks.cpu().numpy(), ks_r)
    np.testing.assert_array_equal(vs.cpu().numpy(), vs_r)
    np.testing.assert_array_equal(kc.cpu().numpy(), kc_r)
    np.testing.assert_array_equal(vc.cpu().numpy(), vc_r)


def test_bridge_fp8_normal_and_strided_output():
    """Normal data: the float32 accumulation may differ from the exact sum by
    at most 64 roundings of 2**-24 on the scale of sum |x w|, which bounds the
    scales and moves a code by at most one step; rows past L stay untouched."""
    say("bridge fp8 normal")
    L, D, n_layers, T = 700, 2048, 2, 1024
    inp = inputs.bridge_inputs(L=L, D=D, n_layers=n_layers, d=256, seed=4, device=DEV)
    k8 = torch.zeros((n_layers, T, 256), dtype=torch.uint8, device=DEV)
    v8 = torch.zeros_like(k8)
    ksc = torch.zeros((n_layers, T), dtype=torch.float32, device=DEV)
    vsc = torch.zeros_like(ksc)
    hs2.hs2_bridge_kv_proj_fp8(inp["x"], inp["w_k"], inp["w_v"], k_out=k8, v_out=v8, k_scale=ksc, v_scale=vsc,
                               out_layer_stride=T * 256, scale_layer_stride=T)
    torch.cuda.synchronize()
    x64, wk64, wv64 = parity.decode(inp["x"]), parity.decode(inp["w_k"]), parity.decode(inp["w_v"])
    k_ref, v_ref = oracle.bridge_kv_proj(x64, wk64, wv64)
    k_abs, v_abs = oracle.bridge_kv_proj(np.abs(x64), np.abs(wk64), np.abs(wv64))
    kc_r, vc_r, ks_r, vs_r = oracle.bridge_kv_proj_fp8(x64, wk64, wv64)
    table = oracle.e4m3_decode_table()
    for codes, sc, ref, mag, codes_r, sc_r in ((k8, ksc, k_ref, k_abs, kc_r, ks_r), (v8, vsc, v_ref, v_abs, vc_r, vs_r)):
        c = codes[:, :L].cpu().numpy()
        s_ = sc[:, :L].cpu().numpy().astype(np.float64)
        slack = 64 * 2.0 ** -24 * mag                     # float32 accumulation error bound per element
        row_slack = slack.max(axis=-1) / 448.0
        assert (np.abs(s_ - sc_r) <= row_slack + 2.0 ** -23 * sc_r).all()
        got = table[c] * s_[..., None]
        # half a step of the value's e4m3 binade (2**-4 relative, 2**-10 scale below the normals),
        # plus one more step where the float32 sum sits on the other side of a rounding boundary
        step = np.maximum(2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref) / s_[..., None], 2.0 ** -6))) - 3),
                          2.0 ** -9) * s_[..., None]
        assert (np.abs(got - ref) <= 1.5 * step + 2 * slack).all()
        assert (c == codes_r).mean() > 0.999
        assert (codes[:, L:] == 0).all() and (sc[:, L:] == 0).all()



# --------------------------------------------------------------------------- maximum selection size
@pytest.mark.parametrize("n_q", [24, 40])   # B * n_q = 48: split sparse form; 80: one workgroup per query
def test_max_selection_size(n_q):
    """window + topk = HS2_MAX_SELECT (4096): the token selection (whose single-read estimate
    cannot keep that many candidates, so the exact path runs), the block selection with 992
    blocks of 4, and the sparse layer over 4096-entry index sets."""
    window, topk, q_pos0 = 128, 3968, 6000
    T = q_pos0 + n_q
    say("max selection", n_q)
    rng = np.random.default_rng(n_q)
    ld = (T + 3) // 4 * 4
    sc = _score_rows(rng, 2, n_q, q_pos0, ld)
    _select_case(sc, q_pos0, T, window, topk)
    s = torch.from_numpy(sc).to(DEV)
    idx_b, cnt_b = hs2.hs2_select_blocks_window(s, q_pos0=q_pos0, T=T, window=window, topk=topk, block=4)
    idx, cnt = hs2.hs2_select_topk_window(s, q_pos0=q_pos0, T=T, window=window, topk=topk)
    inp = inputs.attention_inputs(B=2, n_q=n_q, T=T, H=16, d=256, kv="bf16", n_sparse=1, seed=n_q, device=DEV)
    o, lse = hs2.hs2_sparse_attn_reuse(inp["q_sparse"][0], inp["k"], inp["v"], idx, cnt, sm_scale=SCALE)
    torch.cuda.synchronize()
    idxb_np, cntb_np = idx_b.cpu().numpy(), cnt_b.cpu().numpy()
    idx_np, cnt_np = idx.cpu().numpy(), cnt.cpu().numpy()
    o_ref = np.zeros(tuple(inp["q_sparse"][0].shape))
    lse_ref = np.zeros(o_ref.shape[:3])
    for b in range(2):
        k64, v64 = parity.kv_f64(inp, b)
        q64 = parity.decode(inp["q_sparse"][0][b])
        for i in range(n_q):
            p = q_pos0 + i
            parity.check_block_selection(idxb_np[b, i], int(cntb_np[b, i]), sc[b, i], p, window, topk, 4)
            assert int(cnt_np[b, i]) == window + topk
            o_ref[b, i], lse_ref[b, i] = oracle.sparse_attn_reuse(q64[i], k64, v64, idx_np[b, i, : cnt_np[b, i]], SCALE)
    parity.check_out(o, o_ref, "bf16")
    parity.check_lse(lse, lse_ref)

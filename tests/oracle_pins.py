"""Checks that tie the CPU oracle to facts outside itself.

Each ``pin_*`` function takes the oracle module and raises AssertionError when
it disagrees with a library routine, a closed form, an invariant of the method,
a hand-worked example or a brute-force count.  ``test_oracle_pins.py`` runs them
on the real oracle; ``test_oracle_mutations.py`` runs them on deliberately
broken copies and expects at least one to fail for every planted mistake.
"""

from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _sdpa_reference(q, k, v, q_pos0, scale):
    """torch scaled_dot_product_attention (float64, CPU) with a causal mask."""
    n_q, H, d = q.shape
    T = k.shape[0]
    pos = q_pos0 + np.arange(n_q)
    mask = torch.from_numpy(np.arange(T)[None, :] <= pos[:, None])       # [n_q, T]
    qt = torch.from_numpy(q).permute(1, 0, 2)                            # [H, n_q, d]
    kt = torch.from_numpy(k)[None].expand(H, T, d)
    vt = torch.from_numpy(v)[None].expand(H, T, d)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    logits = scale * (qt @ kt.transpose(1, 2))                           # [H, n_q, T]
    logits = logits.masked_fill(~mask[None], float("-inf"))
    lse = torch.logsumexp(logits, dim=-1)                                # [H, n_q]
    prob = torch.softmax(logits, dim=-1)
    return o.permute(1, 0, 2).numpy(), lse.T.numpy(), prob.permute(1, 0, 2).numpy()


# ---------------------------------------------------------------------------
# full attention with scores
# ---------------------------------------------------------------------------

def pin_attn_vs_torch(orc):
    """O, lse and the probabilities against torch SDPA / logsumexp / softmax."""
    r = _rng(11)
    for (n_q, H, d, T, q_pos0) in [(5, 3, 8, 9, 3), (1, 16, 16, 40, 39), (7, 2, 4, 7, 0)]:
        q = r.standard_normal((n_q, H, d))
        k = r.standard_normal((T, d))
        v = r.standard_normal((T, d))
        scale = 0.37
        o, lse, scores = orc.full_attn_scored(q, k, v, q_pos0, scale)
        o_ref, lse_ref, prob_ref = _sdpa_reference(q, k, v, q_pos0, scale)
        np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-12)
        for i in range(n_q):
            p = q_pos0 + i
            assert scores[i].shape == (p + 1,)
            np.testing.assert_allclose(scores[i], prob_ref[i, :, : p + 1].sum(axis=0), rtol=1e-12, atol=1e-14)


def pin_attn_default_scale(orc):
    """Without an explicit scale the softmax uses 1/sqrt(d)."""
    r = _rng(12)
    q = r.standard_normal((3, 2, 16))
    k = r.standard_normal((6, 16))
    v = r.standard_normal((6, 16))
    o, lse, _ = orc.full_attn_scored(q, k, v, 2)
    o_ref, lse_ref, _ = _sdpa_reference(q, k, v, 2, 0.25)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-12)


def pin_attn_zero_query(orc):
    """q = 0: uniform attention, O = mean of v_0..v_p, lse = ln(p+1), s_j = H/(p+1)."""
    r = _rng(13)
    H, d, T = 4, 8, 10
    q = np.zeros((3, H, d))
    k = r.standard_normal((T, d))
    v = r.standard_normal((T, d))
    o, lse, scores = orc.full_attn_scored(q, k, v, 5, 0.5)
    for i in range(3):
        p = 5 + i
        for h in range(H):
            np.testing.assert_allclose(o[i, h], v[: p + 1].mean(axis=0), rtol=1e-13, atol=1e-14)
            assert abs(lse[i, h] - math.log(p + 1)) < 1e-13
        np.testing.assert_allclose(scores[i], np.full(p + 1, H / (p + 1)), rtol=1e-13)


def pin_attn_one_hot_values(orc):
    """V = identity rows: O_h equals the probability row, so sum_h O_h is the score row."""
    r = _rng(14)
    H, d, T = 3, 8, 8
    q = r.standard_normal((4, H, d))
    k = r.standard_normal((T, d))
    v = np.eye(T, d)
    o, _, scores = orc.full_attn_scored(q, k, v, 3, 0.8)
    for i in range(4):
        p = 3 + i
        np.testing.assert_allclose(o[i].sum(axis=0)[: p + 1], scores[i], rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(o[i, :, p + 1:], 0.0, atol=0)
        np.testing.assert_allclose(o[i].sum(axis=1), np.ones(H), rtol=1e-12)


def pin_attn_two_keys(orc):
    """p = 1: P_1 = 1 / (1 + exp(l_0 - l_1)) per head (logistic closed form)."""
    r = _rng(15)
    H, d = 5, 6
    q = r.standard_normal((1, H, d))
    k = r.standard_normal((2, d))
    v = r.standard_normal((2, d))
    scale = 0.3
    o, lse, scores = orc.full_attn_scored(q, k, v, 1, scale)
    s_exp = 0.0
    for h in range(H):
        l0 = scale * float(q[0, h] @ k[0])
        l1 = scale * float(q[0, h] @ k[1])
        p1 = 1.0 / (1.0 + math.exp(l0 - l1))
        np.testing.assert_allclose(o[0, h], (1 - p1) * v[0] + p1 * v[1], rtol=1e-12, atol=1e-14)
        assert abs(lse[0, h] - (max(l0, l1) + math.log1p(math.exp(-abs(l0 - l1))))) < 1e-12
        s_exp += p1
    np.testing.assert_allclose(scores[0], [H - s_exp, s_exp], rtol=1e-12)


def pin_attn_scores_sum_to_heads(orc):
    """Every score row sums to H (each head's probabilities sum to one)."""
    r = _rng(16)
    H = 6
    q = r.standard_normal((9, H, 8)) * 3
    k = r.standard_normal((30, 8))
    v = r.standard_normal((30, 8))
    _, _, scores = orc.full_attn_scored(q, k, v, 21, 0.5)
    for s in scores:
        assert abs(s.sum() - H) < 1e-12
        assert (s >= 0).all()


def pin_attn_causal(orc):
    """Keys and values after the query position do not matter."""
    r = _rng(17)
    q = r.standard_normal((2, 2, 8))
    k = r.standard_normal((12, 8))
    v = r.standard_normal((12, 8))
    a = orc.full_attn_scored(q, k, v, 4, 0.5)
    k2, v2 = k.copy(), v.copy()
    k2[6:] = 100.0 * r.standard_normal((6, 8))
    v2[6:] = 100.0 * r.standard_normal((6, 8))
    b = orc.full_attn_scored(q, k2, v2, 4, 0.5)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
    for x, y in zip(a[2], b[2]):
        np.testing.assert_array_equal(x, y)
    # and a key before the position does matter
    k3 = k.copy()
    k3[0] += 1.0
    c = orc.full_attn_scored(q, k3, v, 4, 0.5)
    assert not np.allclose(a[2][0], c[2][0])


def pin_attn_shift_invariance(orc):
    """Adding c to every key shifts head h's logits by scale*<q_h, c>: P is unchanged."""
    r = _rng(18)
    q = r.standard_normal((3, 4, 8))
    k = r.standard_normal((9, 8))
    v = r.standard_normal((9, 8))
    c = 2.0 * r.standard_normal(8)
    a = orc.full_attn_scored(q, k, v, 5, 0.6)
    b = orc.full_attn_scored(q, k + c, v, 5, 0.6)
    np.testing.assert_allclose(a[0], b[0], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(b[1] - a[1], 0.6 * (q @ c), rtol=1e-10, atol=1e-12)
    for x, y in zip(a[2], b[2]):
        np.testing.assert_allclose(x, y, rtol=1e-11, atol=1e-14)


def pin_attn_brute_force(orc):
    """Scalar loops with math.exp / math.fsum on tiny inputs."""
    r = _rng(19)
    n_q, H, d, T, q0 = 3, 2, 3, 6, 2
    q = r.standard_normal((n_q, H, d))
    k = r.standard_normal((T, d))
    v = r.standard_normal((T, d))
    scale = 0.9
    o, lse, scores = orc.full_attn_scored(q, k, v, q0, scale)
    for i in range(n_q):
        p = q0 + i
        s_bf = [0.0] * (p + 1)
        for h in range(H):
            l = [scale * math.fsum(q[i, h, t] * k[j, t] for t in range(d)) for j in range(p + 1)]
            big = max(l)
            w = [math.exp(x - big) for x in l]
            z = math.fsum(w)
            for j in range(p + 1):
                s_bf[j] += w[j] / z
            for t in range(d):
                ref = math.fsum(w[j] * v[j, t] for j in range(p + 1)) / z
                assert abs(o[i, h, t] - ref) < 1e-12
            assert abs(lse[i, h] - (big + math.log(z))) < 1e-12
        np.testing.assert_allclose(scores[i], s_bf, rtol=1e-12)


# ---------------------------------------------------------------------------
# selection
# ---------------------------------------------------------------------------

def _count_rank_selection(s, p, window, topk):
    """Independent brute force: a candidate is in the top-k when fewer than
    topk candidates beat it (higher score, or equal score and lower index)."""
    n = p + 1
    n_cand = max(0, n - window)
    chosen = set(range(n_cand, n))
    for j in range(n_cand):
        beaten_by = sum(1 for i in range(n_cand) if s[i] > s[j] or (s[i] == s[j] and i < j))
        if beaten_by < topk:
            chosen.add(j)
    return sorted(chosen)


def pin_select_golden(orc):
    with open(os.path.join(GOLDEN, "select_worked_example.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        idx, count, tau = orc.select_topk_window(np.array(c["scores"]), c["p"], c["window"], c["topk"])
        assert list(idx) == c["expected"], c["name"]
        assert count == len(c["expected"]), c["name"]
        assert tau == c["tau"], c["name"]


def pin_select_brute_force(orc):
    r = _rng(21)
    for trial in range(200):
        window = int(r.integers(1, 5))
        topk = int(r.integers(1, 6))
        p = int(r.integers(0, 16))
        s = r.integers(0, 4, size=p + 1).astype(np.float64) / 4.0   # many ties
        idx, count, _ = orc.select_topk_window(s, p, window, topk)
        ref = _count_rank_selection(s, p, window, topk)
        assert list(idx) == ref, (trial, s, p, window, topk)
        assert count == len(ref)


def pin_select_all_ties(orc):
    """Equal scores: the top-k part is the k lowest candidate indices."""
    for p in [1151, 1152, 1153, 2000, 4095]:
        s = np.full(p + 1, 0.5)
        idx, count, tau = orc.select_topk_window(s, p, 128, 1024)
        expect = sorted(set(range(min(1024, p + 1))) | set(range(max(0, p - 127), p + 1)))
        assert list(idx) == expect
        assert count == min(p + 1, 1152)


def pin_select_invariants(orc):
    """|S| = min(p+1, window+topk), window inside S, strictly ascending, in [0, p]."""
    r = _rng(22)
    for p in [0, 1, 126, 127, 128, 129, 1150, 1151, 1152, 1153, 1279, 1280, 1281, 5000]:
        s = r.random(p + 1)
        idx, count, tau = orc.select_topk_window(s, p, 128, 1024)
        assert count == len(idx) == min(p + 1, 1152)
        assert np.all(np.diff(idx) > 0)
        assert idx[0] >= 0 and idx[-1] == p
        assert set(range(max(0, p - 127), p + 1)) <= set(idx.tolist())
        if tau is not None:
            cand = np.arange(p - 127)
            chosen = np.intersect1d(idx, cand)
            assert len(chosen) == 1024
            assert s[chosen].min() == tau
            others = np.setdiff1d(cand, chosen)
            assert (s[others] <= tau).all()


def pin_select_window_scores_ignored(orc):
    """Scores inside the window never change which candidates are chosen."""
    r = _rng(23)
    p = 3000
    s = r.random(p + 1)
    a, _, _ = orc.select_topk_window(s, p, 128, 1024)
    s2 = s.copy()
    s2[p - 127:] = 1e9
    b, _, _ = orc.select_topk_window(s2, p, 128, 1024)
    np.testing.assert_array_equal(a, b)


def pin_select_blocks_golden(orc):
    with open(os.path.join(GOLDEN, "select_blocks_worked_example.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        idx, count, tau = orc.select_blocks_window(np.array(c["scores"], dtype=np.float32), c["p"], c["window"],
                                                   c["topk"], c["block"])
        assert list(idx) == c["expected"], c["name"]
        assert count == len(c["expected"]), c["name"]
        assert tau == c["tau"], c["name"]


def pin_select_blocks_of_one_are_tokens(orc):
    """Blocks of one token are the token-level selection (pinned on its own above)."""
    r = _rng(24)
    for p in [0, 127, 128, 1151, 1152, 1153, 1300, 2500]:
        s = (r.integers(0, 6, size=p + 1) / 8.0).astype(np.float32)   # many ties
        a = orc.select_blocks_window(s, p, 128, 1024, 1)
        b = orc.select_topk_window(s.astype(np.float64), p, 128, 1024)
        assert list(a[0]) == list(b[0]) and a[1] == b[1], p


def _count_rank_blocks(s, p, window, topk, block):
    """Brute force: exact block sums (math.fsum), block b chosen iff fewer than
    topk // block blocks beat it (higher sum, or equal sum and lower index)."""
    n = p + 1
    n_cand = max(0, n - window)
    if n_cand <= topk:
        return list(range(n))
    nb = -(-n_cand // block)
    sums = [math.fsum(s[j] for j in range(b * block, min(n_cand, (b + 1) * block))) for b in range(nb)]
    out = set(range(n_cand, n))
    for b in range(nb):
        beat = sum(1 for c in range(nb) if sums[c] > sums[b] or (sums[c] == sums[b] and c < b))
        if beat < topk // block:
            out |= set(range(b * block, min(n_cand, (b + 1) * block)))
    return sorted(out)


def pin_select_blocks_brute_force(orc):
    r = _rng(25)
    for trial in range(300):
        block = int(2 ** r.integers(0, 4))
        topk = block * int(r.integers(1, 4))
        window = int(r.integers(1, 5))
        p = int(r.integers(0, 40))
        s = r.integers(0, 4, size=p + 1).astype(np.float64) / 4.0   # exact sums, many ties
        idx, count, _ = orc.select_blocks_window(s.astype(np.float32), p, window, topk, block)
        ref = _count_rank_blocks(s, p, window, topk, block)
        assert list(idx) == ref, (trial, s, p, window, topk, block)
        assert count == len(ref)


def pin_block_score_exact(orc):
    """A block scores the exact sum of its scores.  Float32 arithmetic in any
    order loses the 1 in 2^24 + 1 (float32 keeps 24 significant bits, and the
    tie rounds to the even 2^24); the exact sum keeps it.  Sums of dyadic
    values are exact in every precision and must come back unchanged."""
    assert orc.block_score(np.array([2.0 ** 24, 1.0, 0.0, 0.0], dtype=np.float32)) == 2.0 ** 24 + 1
    assert orc.block_score(np.array([1.0, 2.0 ** 24, 1.0, 0.0], dtype=np.float32)) == 2.0 ** 24 + 2
    # 2^-30 + 1 + 2^-30: float32 keeps neither small term next to 1
    assert orc.block_score(np.array([2.0 ** -30, 1.0, 2.0 ** -30, 0.0], dtype=np.float32)) == 1.0 + 2.0 ** -29
    r = _rng(26)
    x = r.integers(0, 1 << 10, size=64).astype(np.float32) / 1024.0
    assert orc.block_score(x) == float(x.astype(np.float64).sum())
    assert orc.block_score(np.array([0.75], dtype=np.float32)) == 0.75
    assert orc.block_score(np.zeros(8, dtype=np.float32)) == 0.0


def pin_select_blocks_exact_sums_decide(orc):
    """Blocks of 4 whose float32 sums tie but whose exact sums differ by one:
    B0 = [2^24, 0, 0, 0] sums to 2^24, B1 = [2^24, 1, 0, 0] to 2^24 + 1.  With
    one block to keep, the exact sums pick B1; float32 sums (any order) would
    tie and give B0 by the index rule.  A third block of zeros never wins."""
    s = np.array([2.0 ** 24, 0, 0, 0, 2.0 ** 24, 1, 0, 0, 0, 0, 0, 0, 5.0, 5.0], dtype=np.float32)
    idx, count, tau = orc.select_blocks_window(s, 13, 2, 4, 4)
    assert list(idx) == [4, 5, 6, 7, 12, 13] and count == 6
    assert tau == 2.0 ** 24 + 1
    # with the small term moved into B0 the choice flips to B0
    s2 = s.copy()
    s2[1], s2[5] = 1.0, 0.0
    idx2, _, _ = orc.select_blocks_window(s2, 13, 2, 4, 4)
    assert list(idx2) == [0, 1, 2, 3, 12, 13]


def pin_select_blocks_invariants(orc):
    """Window inside S, ascending, the candidates of S are whole blocks (cut at
    the last candidate), and exactly topk // block blocks once there is a cut."""
    r = _rng(27)
    for p in [0, 1, 127, 128, 1151, 1152, 1153, 1200, 1215, 1216, 1217, 4000]:
        s = r.random(p + 1).astype(np.float32)
        idx, count, tau = orc.select_blocks_window(s, p, 128, 1024, 64)
        assert count == len(idx) <= 1152
        assert np.all(np.diff(idx) > 0) and idx[-1] == p
        assert set(range(max(0, p - 127), p + 1)) <= set(idx.tolist())
        n_cand = max(0, p - 127)
        chosen = idx[idx < n_cand]
        if tau is None:
            assert count == p + 1
            continue
        blocks = sorted(set((chosen // 64).tolist()))
        assert len(blocks) == 16
        for b in blocks:
            assert set(range(b * 64, min(n_cand, b * 64 + 64))) <= set(chosen.tolist())
        assert count == 128 + len(chosen)


# ---------------------------------------------------------------------------
# sparse attention over the selected set
# ---------------------------------------------------------------------------

def pin_sparse_vs_torch_mask(orc):
    """Sparse attention equals torch SDPA with a boolean mask of the set."""
    r = _rng(31)
    H, d, T = 4, 8, 40
    q = r.standard_normal((H, d))
    k = r.standard_normal((T, d))
    v = r.standard_normal((T, d))
    sel = np.sort(r.choice(T, size=13, replace=False))
    o, lse = orc.sparse_attn_reuse(q, k, v, sel, 0.45)
    mask = torch.zeros(T, dtype=torch.bool)
    mask[torch.from_numpy(sel)] = True
    qt = torch.from_numpy(q)[:, None, :]
    o_ref = torch.nn.functional.scaled_dot_product_attention(
        qt, torch.from_numpy(k)[None].expand(H, T, d), torch.from_numpy(v)[None].expand(H, T, d),
        attn_mask=mask[None, None, :].expand(H, 1, T), scale=0.45)[:, 0]
    np.testing.assert_allclose(o, o_ref.numpy(), rtol=1e-12, atol=1e-12)
    lg = 0.45 * (torch.from_numpy(q) @ torch.from_numpy(k).T)
    lse_ref = torch.logsumexp(lg.masked_fill(~mask[None], float("-inf")), dim=-1)
    np.testing.assert_allclose(lse, lse_ref.numpy(), rtol=1e-12, atol=1e-12)


def pin_sparse_equals_full_when_all_selected(orc):
    """For p+1 <= window+topk the set is [0, p] and the sparse output is full attention."""
    r = _rng(32)
    H, d, T = 3, 8, 50
    q = r.standard_normal((5, H, d))
    k = r.standard_normal((T, d))
    v = r.standard_normal((T, d))
    o_full, lse_full, scores = orc.full_attn_scored(q, k, v, 20, 0.5)
    for i in range(5):
        p = 20 + i
        sel, count, _ = orc.select_topk_window(scores[i], p, 128, 1024)
        o, lse = orc.sparse_attn_reuse(q[i], k, v, sel, 0.5)
        np.testing.assert_allclose(o, o_full[i], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse, lse_full[i], rtol=1e-12, atol=1e-13)


def pin_sparse_order_invariance(orc):
    """The order in which the set is listed does not matter."""
    r = _rng(33)
    q = r.standard_normal((2, 8))
    k = r.standard_normal((30, 8))
    v = r.standard_normal((30, 8))
    sel = r.choice(30, size=11, replace=False)
    a = orc.sparse_attn_reuse(q, k, v, np.sort(sel), 0.5)
    b = orc.sparse_attn_reuse(q, k, v, sel[::-1].copy(), 0.5)
    np.testing.assert_allclose(a[0], b[0], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(a[1], b[1], rtol=1e-13, atol=1e-14)


def pin_sparse_single_and_empty(orc):
    r = _rng(34)
    q = r.standard_normal((3, 4))
    k = r.standard_normal((5, 4))
    v = r.standard_normal((5, 4))
    o, lse = orc.sparse_attn_reuse(q, k, v, np.array([2]), 1.0)
    np.testing.assert_allclose(o, np.tile(v[2], (3, 1)), rtol=0, atol=0)
    np.testing.assert_allclose(lse, q @ k[2], rtol=1e-13)
    o, lse = orc.sparse_attn_reuse(q, k, v, np.array([], dtype=np.int64), 1.0)
    assert (o == 0).all() and np.isneginf(lse).all()


# ---------------------------------------------------------------------------
# KV Bridging projection
# ---------------------------------------------------------------------------

def pin_bridge_integer_exact(orc):
    """Integer-valued inputs: the product equals exact int64 matrix products."""
    r = _rng(41)
    L, D, d, n = 7, 12, 5, 3
    x = r.integers(-8, 9, size=(L, D))
    wk = r.integers(-4, 5, size=(n, D, d))
    wv = r.integers(-4, 5, size=(n, D, d))
    k, v = orc.bridge_kv_proj(x.astype(np.float64), wk.astype(np.float64), wv.astype(np.float64))
    for m in range(n):
        np.testing.assert_array_equal(k[m], (x @ wk[m]).astype(np.float64))
        np.testing.assert_array_equal(v[m], (x @ wv[m]).astype(np.float64))


def pin_bridge_brute_force(orc):
    r = _rng(42)
    L, D, d, n = 3, 4, 2, 2
    x = r.standard_normal((L, D))
    wk = r.standard_normal((n, D, d))
    wv = r.standard_normal((n, D, d))
    k, v = orc.bridge_kv_proj(x, wk, wv)
    for m, i, j in itertools.product(range(n), range(L), range(d)):
        assert abs(k[m, i, j] - math.fsum(x[i, t] * wk[m, t, j] for t in range(D))) < 1e-13
        assert abs(v[m, i, j] - math.fsum(x[i, t] * wv[m, t, j] for t in range(D))) < 1e-13


# ---------------------------------------------------------------------------
# storage formats
# ---------------------------------------------------------------------------

def pin_bf16_decode(orc):
    bits = np.arange(0, 65536, 7, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = orc.bf16_bits_to_f64(bits)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def pin_bf16_round(orc):
    r = _rng(51)
    x = np.concatenate([r.standard_normal(20000) * 10.0 ** r.integers(-30, 30, 20000),
                        r.standard_normal(1000)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(orc.f64_to_bf16_bits(x.astype(np.float64)), ref)
    # hand-checked halfway cases (8 significant bits: the step above 1 is 2**-7)
    cases = {1.0 + 2.0 ** -8: 0x3F80, 1.0 + 3 * 2.0 ** -8: 0x3F82,
             -(1.0 + 2.0 ** -8 + 2.0 ** -30): 0xBF81, 2.0 ** -133: 0x0001, 3.0 * 2.0 ** -134: 0x0002,
             3.4e38: 0x7F80, 3.3e38: 0x7F78}
    for val, want in cases.items():
        assert int(orc.f64_to_bf16_bits(np.array([val]))[0]) == want, val


def pin_e4m3_table(orc):
    t = orc.e4m3_decode_table()
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(t), np.isnan(ref))
    assert np.array_equal(t[~np.isnan(t)], ref[~np.isnan(ref)])
    assert t[0x7E] == 448.0 and t[0x01] == 2.0 ** -9 and t[0x08] == 2.0 ** -6
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF]) and np.isnan(t).sum() == 2


def pin_decode_rows(orc):
    codes = np.array([[0x38, 0xB8], [0x40, 0x01]], dtype=np.uint8)   # 1, -1 ; 2, 2**-9
    scale = np.array([0.5, 4.0], dtype=np.float32)
    np.testing.assert_array_equal(orc.decode_rows(codes, "e4m3", scale), [[0.5, -0.5], [8.0, 2.0 ** -7]])
    np.testing.assert_array_equal(orc.decode_rows(np.array([0x3F80, 0xC000], dtype=np.uint16), "bf16"), [1.0, -2.0])


# ---------------------------------------------------------------------------
# FP8 e4m3 cache rows
# ---------------------------------------------------------------------------

def pin_e4m3_encode_vs_torch(orc):
    """Encoding against torch's float8_e4m3fn conversion (round to nearest even):
    every finite code's own value, every midpoint between neighbours (the ties),
    and random values over the whole range and near the subnormals."""
    t = orc.e4m3_decode_table()
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    np.testing.assert_array_equal(orc.f64_to_e4m3_codes(t[finite]), finite.astype(np.uint8))
    pos = np.unique(t[:0x7F])
    mid = (pos[:-1] + pos[1:]) / 2
    r = _rng(61)
    y = np.concatenate([mid, -mid, r.uniform(-448, 448, 5000), r.uniform(-0.03, 0.03, 5000)]).astype(np.float32)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(orc.f64_to_e4m3_codes(y.astype(np.float64)), ref)


def pin_e4m3_encode_hand(orc):
    # ties go to the even 3-bit mantissa; the sign bit follows the sign (also of zero)
    cases = [(1.0 + 1 / 16, 0x38), (1.0 + 3 / 16, 0x3A), (-(1.0 + 1 / 16), 0xB8), (448.0, 0x7E), (416.0, 0x7D),
             (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02), (2.0 ** -6, 0x08), (0.0, 0x00), (-0.0, 0x80),
             (-2.0 ** -12, 0x80)]
    for val, want in cases:
        assert int(orc.f64_to_e4m3_codes(np.array([val]))[0]) == want, val


def pin_bridge_fp8_closed_form(orc):
    """One-hot hidden states select weight rows: a row [4, -2, 1, 0, ...] has
    amax 4, scale fl32(4/448) and codes for 448, -224, 112, 0; a zero row keeps
    scale 1 and codes 0."""
    D, d = 3, 8
    x = np.array([[1.0, 0.0, 0.0], [0.0, 0.0, 0.0]])
    wk = np.zeros((1, D, d))
    wk[0, 0, :4] = [4.0, -2.0, 1.0, 0.0]
    wv = np.zeros((1, D, d))
    wv[0, 0, 5] = -3.0
    kc, vc, ks, vs = orc.bridge_kv_proj_fp8(x, wk, wv)
    assert ks.dtype == np.float32 and kc.dtype == np.uint8
    assert ks[0, 0] == np.float32(4.0 / 448.0) and ks[0, 1] == 1.0 and vs[0, 1] == 1.0
    np.testing.assert_array_equal(kc[0, 0, :4], [0x7E, 0xF6, 0x6E, 0x00])
    assert (kc[0, 1] == 0).all() and (vc[0, 1] == 0).all()
    assert vs[0, 0] == np.float32(3.0 / 448.0) and vc[0, 0, 5] == 0xFE and (np.delete(vc[0, 0], 5) == 0).all()


def pin_bridge_fp8_divides_by_the_scale(orc):
    """Rows whose quotients land on an e4m3 tie: 39 * 448 / 52 is exactly 336,
    halfway between the codes for 320 and 352.  The float32 quotient
    fl32(39 / fl32(52/448)) is 336.0 and rounds to the even 320 (0x7A);
    multiplying by fl32(448/52) instead would give 336.00003 and 352 (0x7B).
    For amax 124 and 93 it is the other way round: the quotient is 336.00003
    (352, 0x7B) where the reciprocal product gives 336.0 (320, 0x7A).  The
    largest element always maps to 448 (0x7E) and signs carry over (0x80)."""
    D, d = 2, 4
    x = np.array([[1.0, 0.0], [0.0, 1.0]])
    wk = np.zeros((1, D, d))
    wk[0, 0, :2] = [52.0, 39.0]
    wk[0, 1, :3] = [-124.0, -93.0, 93.0]
    wv = np.zeros((1, D, d))
    wv[0, 0, :2] = [124.0, 93.0]
    wv[0, 1, :2] = [52.0, -39.0]
    kc, vc, ks, vs = orc.bridge_kv_proj_fp8(x, wk, wv)
    np.testing.assert_array_equal(kc[0, 0], [0x7E, 0x7A, 0x00, 0x00])
    np.testing.assert_array_equal(kc[0, 1], [0xFE, 0xFB, 0x7B, 0x00])
    np.testing.assert_array_equal(vc[0, 0], [0x7E, 0x7B, 0x00, 0x00])
    np.testing.assert_array_equal(vc[0, 1], [0x7E, 0xFA, 0x00, 0x00])
    assert ks[0, 0] == np.float32(np.float32(52.0) / np.float32(448.0)) and vs[0, 0] == np.float32(124.0 / 448.0)


def pin_bridge_fp8_dequant_bound(orc):
    """decode(code) * scale is within half an e4m3 step of the projection: 2**-4
    relative for normal codes, 2**-10 * scale absolute below them."""
    r = _rng(62)
    L, D, d, n = 9, 40, 16, 2
    x = r.standard_normal((L, D))
    wk = r.standard_normal((n, D, d)) * 0.02
    wv = r.standard_normal((n, D, d)) * 0.02
    k, v = orc.bridge_kv_proj(x, wk, wv)
    kc, vc, ks, vs = orc.bridge_kv_proj_fp8(x, wk, wv)
    t = orc.e4m3_decode_table()
    for ref, codes, sc in ((k, kc, ks), (v, vc, vs)):
        got = t[codes] * sc.astype(np.float64)[..., None]
        bound = (2.0 ** -4 * np.abs(ref) + 2.0 ** -10 * sc.astype(np.float64)[..., None]) * (1 + 1e-6)
        assert (np.abs(got - ref) <= bound).all()
        # the largest element of each row lands on +-448
        amax_pos = np.abs(ref).argmax(axis=-1)
        top = np.take_along_axis(codes, amax_pos[..., None], axis=-1)[..., 0]
        assert np.isin(top, [0x7E, 0xFE]).all()


# ---------------------------------------------------------------------------
# self-decoder sliding-window attention with partial rotary embedding
# ---------------------------------------------------------------------------

def _rope_complex(x, pos, R, base):
    """RoPE in its complex form: the pair (x[2m], x[2m+1]) is the complex number
    x[2m] + i x[2m+1], multiplied by exp(i t base^(-2m/R)); other dims untouched."""
    x = np.array(x, dtype=np.float64)
    if R == 0:
        return x
    z = x[..., 0:R:2] + 1j * x[..., 1:R:2]
    w = np.exp(1j * np.outer(np.asarray(pos, dtype=np.float64), base ** (-np.arange(R // 2) * 2.0 / R)))
    z = z * w
    x[..., 0:R:2] = z.real
    x[..., 1:R:2] = z.imag
    return x


def pin_rope_complex_form(orc):
    """rope_partial against the complex-multiplication form, at small and large positions."""
    r = _rng(71)
    for R, base in [(2, 10000.0), (8, 100.0), (64, 10000.0), (256, 500000.0)]:
        x = r.standard_normal((3, 7, 256))
        pos = np.array([0, 1, 2, 127, 131071, 1 << 20, 40000])
        np.testing.assert_allclose(orc.rope_partial(x, pos, R, base), _rope_complex(x, pos, R, base),
                                   rtol=1e-9, atol=1e-9)
    x = r.standard_normal((4, 256))
    np.testing.assert_array_equal(orc.rope_partial(x, np.arange(4), 0), x)


def pin_rope_closed_forms(orc):
    """Exact rotations: position 0 is the identity; with base = (2/pi)^2 and R = 4
    the second pair turns by pi/2 at position 1 ((a, b) -> (-b, a)) and by pi at
    position 2; the first pair always turns by t radians; dims >= R stay."""
    x = np.array([[3.0, 5.0, 7.0, 11.0, 13.0, 17.0]] * 3)
    base = (2.0 / math.pi) ** 2
    y = orc.rope_partial(x, np.array([0, 1, 2]), 4, base)
    np.testing.assert_array_equal(y[0], x[0])
    np.testing.assert_allclose(y[1, 2:4], [-11.0, 7.0], atol=1e-12)
    np.testing.assert_allclose(y[2, 2:4], [-7.0, -11.0], atol=1e-12)
    np.testing.assert_allclose(y[1, 0:2], [3 * math.cos(1) - 5 * math.sin(1), 3 * math.sin(1) + 5 * math.cos(1)],
                               atol=1e-12)
    np.testing.assert_array_equal(y[:, 4:], x[:, 4:])
    # a rotation keeps each pair's length
    r = _rng(72)
    z = r.standard_normal((5, 64))
    w = orc.rope_partial(z, np.arange(5) * 999, 64, 10000.0)
    np.testing.assert_allclose(w[:, 0::2] ** 2 + w[:, 1::2] ** 2, z[:, 0::2] ** 2 + z[:, 1::2] ** 2, rtol=1e-12)


def pin_swa_window_of_one(orc):
    """window = 1: o = v_p, and lse = scale <q, k_p> (q and k_p are turned by the
    same angle, which leaves their inner product unchanged)."""
    r = _rng(73)
    H, d, T = 3, 16, 20
    q = r.standard_normal((4, H, d))
    k = r.standard_normal((T, d))
    v = r.standard_normal((T, d))
    o, lse = orc.swa_attn(q, k, v, 9, window=1, rope_dims=8, base=10.0, sm_scale=0.3)
    for i in range(4):
        p = 9 + i
        np.testing.assert_allclose(o[i], np.tile(v[p], (H, 1)), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse[i], 0.3 * (q[i] @ k[p]), rtol=1e-10, atol=1e-12)


def pin_swa_full_window_is_full_attention(orc):
    """Without rotation and with a window covering every key, SWA is full attention."""
    r = _rng(74)
    q = r.standard_normal((6, 2, 8))
    k = r.standard_normal((15, 8))
    v = r.standard_normal((15, 8))
    o, lse = orc.swa_attn(q, k, v, 9, window=100, rope_dims=0, sm_scale=0.5)
    o_ref, lse_ref, _ = _sdpa_reference(q, k, v, 9, 0.5)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-12)


def pin_swa_vs_torch_band_mask(orc):
    """torch SDPA with a band mask on queries and keys rotated by the complex form."""
    r = _rng(75)
    n_q, H, d, T, q0, W, R, base = 9, 4, 32, 40, 25, 6, 16, 50.0
    q = r.standard_normal((n_q, H, d))
    k = r.standard_normal((T, d))
    v = r.standard_normal((T, d))
    o, lse = orc.swa_attn(q, k, v, q0, window=W, rope_dims=R, base=base, sm_scale=0.2)
    pos = q0 + np.arange(n_q)
    qr = _rope_complex(np.swapaxes(q, 0, 1), pos, R, base)            # [H, n_q, d]
    kr = _rope_complex(k, np.arange(T), R, base)
    keys = np.arange(T)
    mask = torch.from_numpy((keys[None, :] <= pos[:, None]) & (keys[None, :] > pos[:, None] - W))
    qt = torch.from_numpy(qr)
    kt = torch.from_numpy(kr)[None].expand(H, T, d)
    vt = torch.from_numpy(v)[None].expand(H, T, d)
    o_ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=0.2)
    lg = (0.2 * (qt @ kt.transpose(1, 2))).masked_fill(~mask[None], float("-inf"))
    np.testing.assert_allclose(o, o_ref.permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse, torch.logsumexp(lg, dim=-1).T.numpy(), rtol=1e-10, atol=1e-12)


def pin_swa_window_edges(orc):
    """Keys before p-W+1 and after p do not matter; the oldest key inside does."""
    r = _rng(76)
    H, d, T, W = 2, 16, 30, 5
    q = r.standard_normal((3, H, d))
    k = r.standard_normal((T, d))
    v = r.standard_normal((T, d))
    a = orc.swa_attn(q, k, v, 12, window=W, rope_dims=8)
    k2, v2 = k.copy(), v.copy()
    k2[:8] = 50 * r.standard_normal((8, d))      # before the first window (12 - 5 + 1 = 8)
    v2[:8] = 50 * r.standard_normal((8, d))
    k2[15:] = 50 * r.standard_normal((T - 15, d))  # after the last query (14)
    b = orc.swa_attn(q, k2, v2, 12, window=W, rope_dims=8)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
    k3 = k.copy()
    k3[8] += 1.0                                  # the oldest key of the first query's window
    c = orc.swa_attn(q, k3, v, 12, window=W, rope_dims=8)
    assert not np.allclose(a[1][0], c[1][0])


def pin_swa_relative_positions(orc):
    """Moving the whole sequence c positions later (c unseen keys in front)
    leaves every result unchanged: rotated logits depend on position differences."""
    r = _rng(77)
    H, d, T, W, c = 2, 64, 24, 7, 1000
    q = r.standard_normal((5, H, d))
    k = r.standard_normal((T, d))
    v = r.standard_normal((T, d))
    a = orc.swa_attn(q, k, v, 15, window=W, rope_dims=64, base=10000.0)
    pad = r.standard_normal((c, d))
    b = orc.swa_attn(q, np.concatenate([pad, k]), np.concatenate([pad, v]), 15 + c, window=W, rope_dims=64,
                     base=10000.0)
    np.testing.assert_allclose(a[0], b[0], rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(a[1], b[1], rtol=1e-9, atol=1e-11)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]

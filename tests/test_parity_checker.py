"""The acceptance checker itself, on the CPU: it passes outputs that carry only
the rounding a correct bf16 kernel makes, and it fails a planted gather
mistake in long index sets that a bound scaled by the batch maximum let
through (rows of long sets have small |O|)."""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import parity  # noqa: E402

import oracle  # noqa: E402
from token_level_sparse_full_amd import inputs  # noqa: E402

SIZES = [0, 1, 5, 31, 32, 33, 100, 1152, 700, 17]


def _bf16_round(x):
    return oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits(x))


@pytest.fixture(scope="module")
def case():
    B, n_q, T, H = 1, 20, 3000, 16
    inp = inputs.attention_inputs(B=B, n_q=n_q, T=T, H=H, d=256, kv="bf16", n_sparse=0, seed=11, device="cpu")
    rng = np.random.default_rng(5)
    sets = [np.sort(rng.choice(T, size=SIZES[i % len(SIZES)], replace=False)) for i in range(n_q)]
    q = parity.decode(inp["q"][0])
    k, v = parity.kv_f64(inp, 0)
    o_ref = np.stack([oracle.sparse_attn_reuse(q[i], k, v, sets[i], 1 / 16)[0] for i in range(n_q)])
    return q, k, v, sets, o_ref


def test_rounded_reference_passes(case):
    q, k, v, sets, o_ref = case
    parity.check_out(_bf16_round(o_ref), o_ref, "bf16")


def test_wrong_value_rows_of_one_piece_fail(case):
    """V rows of the second 128-key piece of every set of 256 or more keys come
    from the neighbouring key: lse is unchanged (the K side is right), and the
    error stays below 2**-5 of the batch's largest |O| -- the row-wise bound
    must still catch it."""
    q, k, v, sets, o_ref = case
    o_bad = o_ref.copy()
    for i, sel in enumerate(sets):
        if sel.size >= 256:
            v_bad = v.copy()
            v_bad[sel[128:256]] = v[(sel[128:256] + 1) % v.shape[0]]
            o_bad[i] = oracle.sparse_attn_reuse(q[i], k, v_bad, sel, 1 / 16)[0]
    o_bad = _bf16_round(o_bad)
    batch_err = np.abs(o_bad - o_ref).max()
    assert batch_err < 2.0 ** -5 * np.abs(o_ref).max()        # what a batch-wide bound would accept
    with pytest.raises(AssertionError, match="rows off"):
        parity.check_out(o_bad, o_ref, "bf16")


def test_zero_rows_must_stay_zero(case):
    q, k, v, sets, o_ref = case
    empty = [i for i, s in enumerate(sets) if s.size == 0]
    assert empty
    o_bad = o_ref.copy()
    o_bad[empty[0], 3, 7] = 1e-4
    with pytest.raises(AssertionError):
        parity.check_out(o_bad, o_ref, "bf16")


def _f32_tree_selection(s, p, window, topk, block):
    """Block selection ranked on float32 pairwise-tree sums (what a kernel
    that adds in float32 does), built here only to exercise the checker."""
    n_cand = p + 1 - window
    nb = -(-n_cand // block)
    pad = np.zeros(nb * block, dtype=np.float32)
    pad[:n_cand] = s[:n_cand]
    t = pad.reshape(nb, block)
    while t.shape[1] > 1:
        t = (t[:, 0::2] + t[:, 1::2]).astype(np.float32)
    order = sorted(range(nb), key=lambda b: (-float(t[b, 0]), b))[: topk // block]
    toks = [np.arange(b * block, min(n_cand, (b + 1) * block)) for b in order]
    sel = np.sort(np.concatenate(toks + [np.arange(n_cand, p + 1)]))
    out = np.full(window + topk, -1, dtype=np.int32)
    out[: sel.size] = sel
    return out, sel.size


@pytest.mark.parametrize("block", [4, 64, 256])
def test_block_checker_accepts_float32_tree_sums(block):
    rng = np.random.default_rng(block)
    p, window, topk = 9000, 128, 1024
    swaps = 0
    for trial in range(6):
        s = (rng.lognormal(0.0, 3.0, p + 1) / (p + 1)).astype(np.float32)
        if trial % 2:   # near-ties: many blocks share the same sum up to float32 rounding
            s = (np.float32(1.0 / 4096) * (1 + rng.integers(0, 4, p + 1) * np.float32(2 ** -22))).astype(np.float32)
        idx, cnt = _f32_tree_selection(s, p, window, topk, block)
        swaps += parity.check_block_selection(idx, cnt, s, p, window, topk, block)


def test_block_checker_rejects_a_wrong_block():
    rng = np.random.default_rng(7)
    p, window, topk, block = 5000, 128, 1024, 64
    s = rng.random(p + 1).astype(np.float32)
    idx, cnt = _f32_tree_selection(s, p, window, topk, block)
    n_cand = p + 1 - window
    chosen = np.unique(idx[: cnt][idx[: cnt] < n_cand] // block)
    worst = min(set(range(n_cand // block)) - set(chosen.tolist()),
                key=lambda b: s[b * block:(b + 1) * block].astype(np.float64).sum())
    bad_blocks = np.sort(np.concatenate([chosen[1:], [worst]]))
    sel = np.sort(np.concatenate([np.arange(b * block, (b + 1) * block) for b in bad_blocks] +
                                 [np.arange(n_cand, p + 1)]))
    bad = np.full(window + topk, -1, dtype=np.int32)
    bad[: sel.size] = sel
    with pytest.raises(AssertionError, match="outside the band"):
        parity.check_block_selection(bad, sel.size, s, p, window, topk, block)

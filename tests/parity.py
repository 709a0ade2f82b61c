"""Helpers for the GPU parity tests: run the oracle on the very bytes the HIP
path consumed and compare with the acceptance rules.

Acceptance (stated once here, used by every GPU test):
* attention outputs: max |O_gpu - O_ref| <= 2e-2 for bf16 inputs and <= 1e-4 for
  float32 inputs; additionally (tighter, derived from the arithmetic) every
  output row (one query and head) must be within 2**-5 (bf16 and e4m3) or 1e-4
  (float32) of that row's own max |O_ref|, plus a floor of 2**-24 of the
  largest |O_ref| in the batch for rows that are 0.  P and O are rounded to
  bf16 (2**-9 relative each), so a correct kernel sits near 2**-8 of each row;
  a row-wise bound keeps the rows of long sets, whose |O| is small, as tightly
  checked as the short ones;
* lse: |lse_gpu - lse_ref| <= 1e-4 (float32 exp2/log2 of exact logits);
* scores: |s_gpu - s_ref| <= 1e-5 * s_ref + 1e-12 (float32 logits of exact bf16
  products, v_exp_f32 accuracy ~1 ulp: a correct kernel is near 1e-6 relative);
* selections: |S_gpu| = |S_ref| = min(p+1, window+topk); the window is inside;
  strictly ascending within [0, p]; every index in the symmetric difference has
  a reference score within 1e-5 * tau of the reference cut score tau (ties at
  the cut resolve to the lower index, so with identical float32 scores the sets
  must be equal);
* block-level selections (scored on exact block sums by the oracle): the
  selected candidates are whole blocks, exactly topk / block of them, the
  window is inside and the count matches; every block in the symmetric
  difference with the oracle's blocks has an exact sum within BLOCK_BAND(block)
  * tau of the oracle's cut sum tau.  The kernel adds a block's block <= 256
  non-negative float32 scores as a pairwise tree of depth t = log2(block), so
  its sum is within g = t u / (1 - t u) (u = 2**-24) of the exact sum, relative;
  two blocks can change places only when both exact sums lie within
  2 g / (1 - g) of tau.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
from token_level_sparse_full_amd import inputs

O_TOL = {"bf16": 2e-2, "f32": 1e-4, "e4m3": 2e-2}
O_REL = {"bf16": 2.0 ** -5, "f32": 1e-4, "e4m3": 2.0 ** -5}
LSE_TOL = 1e-4
S_REL = 1e-5
TAU_REL = 1e-5


def BLOCK_BAND(block: int) -> float:
    t = max(1, int(block).bit_length() - 1)
    u = 2.0 ** -24
    g = t * u / (1 - t * u)
    return 2 * g / (1 - g)


def decode(t: torch.Tensor, scale: torch.Tensor | None = None) -> np.ndarray:
    kind = inputs.kind_of(t)
    return oracle.decode_rows(inputs.raw_numpy(t), kind, inputs.raw_numpy(scale))


def kv_f64(inp: dict, b: int):
    ks = None if inp["k_scale"] is None else inp["k_scale"][b]
    vs = None if inp["v_scale"] is None else inp["v_scale"][b]
    return decode(inp["k"][b], ks), decode(inp["v"][b], vs)


def check_out(o_gpu, o_ref: np.ndarray, kind: str, what: str = "o"):
    """o_gpu (a tensor or an array) against o_ref [..., d]; every row along the
    last axis is bounded by its own magnitude.  Returns the max abs error."""
    if isinstance(o_gpu, torch.Tensor):
        o_gpu = o_gpu.detach().float().cpu().numpy()
    g = np.asarray(o_gpu, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    assert g.shape == o_ref.shape, (g.shape, o_ref.shape)
    diff = np.abs(g - o_ref)
    err = diff.max()
    assert err <= O_TOL[kind], f"{what}: max abs err {err:.3e} > {O_TOL[kind]}"
    row_err = diff.max(axis=-1)
    row_max = np.abs(o_ref).max(axis=-1)
    bound = O_REL[kind] * row_max + 2.0 ** -24 * np.abs(o_ref).max()
    bad = row_err > bound
    if bad.any():
        w = np.unravel_index(np.argmax(np.where(bad, row_err / np.maximum(bound, 1e-300), 0)), bad.shape)
        raise AssertionError(f"{what}: {bad.sum()} rows off; row {w}: err {row_err[w]:.3e} vs max|ref| "
                             f"{row_max[w]:.3e} (bound {bound[w]:.3e})")
    return err


def check_lse(lse_gpu: torch.Tensor, lse_ref: np.ndarray):
    g = lse_gpu.detach().cpu().numpy().astype(np.float64)
    err = np.abs(g - lse_ref).max()
    assert err <= LSE_TOL, f"lse err {err:.3e}"
    return err


def scores_rel_for_logits(max_logit_log2: float) -> float:
    """Relative score bound when logits reach max_logit_log2 (log2 units) in magnitude: a
    probability is exp2(x - lse2), and x and lse2 are float32 values of that magnitude, each
    within about two units in the last place of the exact ones (the logit from a float32 dot
    product, the lse from m + log2(z)), so the exponent alone may be off by 4 ulps of it."""
    return S_REL + 4.0 * math.log(2.0) * 2.0 ** -24 * max(1.0, abs(max_logit_log2))


def check_scores(s_gpu: np.ndarray, s_ref: np.ndarray, what: str = "scores", rel: float = S_REL):
    err = np.abs(s_gpu.astype(np.float64) - s_ref)
    bad = err > rel * s_ref + 1e-12
    assert not bad.any(), f"{what}: {bad.sum()} entries off, worst rel {(err / np.maximum(s_ref, 1e-30)).max():.3e}"
    return (err / np.maximum(s_ref, 1e-30)).max()


def check_selection(idx_gpu: np.ndarray, count_gpu: int, s_ref: np.ndarray, p: int, window: int = 128,
                    topk: int = 1024, exact: bool = False):
    """Selection of the query at position p against the oracle's, on the oracle's scores."""
    ref, n_ref, tau = oracle.select_topk_window(s_ref, p, window, topk)
    assert count_gpu == n_ref == min(p + 1, window + topk), (count_gpu, n_ref, p)
    got = np.asarray(idx_gpu[:count_gpu], dtype=np.int64)
    assert (np.asarray(idx_gpu[count_gpu:]) == -1).all(), "padding must be -1"
    assert np.all(np.diff(got) > 0), "indices must be strictly ascending"
    assert got[0] >= 0 and got[-1] <= p
    win = np.arange(max(0, p - window + 1), p + 1)
    assert np.isin(win, got).all(), "window not fully selected"
    diff = np.setxor1d(got, ref)
    if exact or tau is None:
        assert diff.size == 0, f"selection differs at {diff[:10]}"
        return 0
    off = np.abs(s_ref[diff] - tau) > TAU_REL * tau
    assert not off.any(), f"swaps outside the boundary band: {diff[off][:10]} (tau={tau})"
    return diff.size


def check_block_selection(idx_gpu: np.ndarray, count_gpu: int, s: np.ndarray, p: int, window: int, topk: int,
                          block: int):
    """Block-level selection of the query at position p against the oracle's,
    on the float32 scores s the GPU selected from.  Returns the number of
    blocks swapped within the band."""
    s = np.asarray(s, dtype=np.float64)[: p + 1]
    ref, n_ref, tau = oracle.select_blocks_window(s, p, window, topk, block)
    got = np.asarray(idx_gpu[:count_gpu], dtype=np.int64)
    assert (np.asarray(idx_gpu[count_gpu:]) == -1).all(), "padding must be -1"
    assert count_gpu >= 1 and np.all(np.diff(got) > 0), "indices must be strictly ascending"
    assert got[0] >= 0 and got[-1] <= p
    if tau is None:
        assert count_gpu == n_ref and np.array_equal(got, ref), "every key must be selected"
        return 0
    n_cand = p + 1 - window
    assert np.array_equal(got[got >= n_cand], np.arange(n_cand, p + 1)), "window not exactly selected"
    cand = got[got < n_cand]
    blocks = np.unique(cand // block)
    assert blocks.size == topk // block, f"{blocks.size} blocks selected, want {topk // block}"
    whole = np.concatenate([np.arange(b * block, min(n_cand, (b + 1) * block)) for b in blocks])
    assert np.array_equal(cand, whole), "selected blocks must be whole"
    ref_blocks = np.unique(ref[ref < n_cand] // block)
    diff = np.setxor1d(blocks, ref_blocks)
    for b in diff:
        sig = oracle.block_score(s[b * block: min(n_cand, (b + 1) * block)])
        assert abs(sig - tau) <= BLOCK_BAND(block) * tau, \
            f"block {b} (sum {sig!r}) swapped outside the band of tau {tau!r}"
    return diff.size // 2

"""Helpers for the GPU parity tests: run the oracle on the very bytes the HIP
path consumed and compare with the acceptance rules.

Acceptance (stated once here, used by every GPU test):
* attention outputs: max |O_gpu - O_ref| <= 2e-2 for bf16 inputs and <= 1e-4 for
  float32 inputs; additionally (tighter, derived from the arithmetic) the error
  relative to max |O_ref| must stay below 2**-5 for bf16 (P and O are rounded to
  bf16, 2**-9 relative each, so a correct kernel sits near 2**-8) and below 1e-4
  for float32;
* lse: |lse_gpu - lse_ref| <= 1e-4 (float32 exp2/log2 of exact logits);
* scores: |s_gpu - s_ref| <= 1e-5 * s_ref + 1e-12 (float32 logits of exact bf16
  products, v_exp_f32 accuracy ~1 ulp: a correct kernel is near 1e-6 relative);
* selections: |S_gpu| = |S_ref| = min(p+1, window+topk); the window is inside;
  strictly ascending within [0, p]; every index in the symmetric difference has
  a reference score within 1e-5 * tau of the reference cut score tau (ties at
  the cut resolve to the lower index, so with identical float32 scores the sets
  must be equal).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from token_level_sparse_full_amd import inputs

O_TOL = {"bf16": 2e-2, "f32": 1e-4, "e4m3": 2e-2}
O_REL = {"bf16": 2.0 ** -5, "f32": 1e-4, "e4m3": 2.0 ** -5}
LSE_TOL = 1e-4
S_REL = 1e-5
TAU_REL = 1e-5


def decode(t: torch.Tensor, scale: torch.Tensor | None = None) -> np.ndarray:
    kind = inputs.kind_of(t)
    return oracle.decode_rows(inputs.raw_numpy(t), kind, inputs.raw_numpy(scale))


def kv_f64(inp: dict, b: int):
    ks = None if inp["k_scale"] is None else inp["k_scale"][b]
    vs = None if inp["v_scale"] is None else inp["v_scale"][b]
    return decode(inp["k"][b], ks), decode(inp["v"][b], vs)


def check_out(o_gpu: torch.Tensor, o_ref: np.ndarray, kind: str, what: str = "o"):
    g = o_gpu.detach().float().cpu().numpy().astype(np.float64)
    err = np.abs(g - o_ref).max()
    ref_max = np.abs(o_ref).max()
    assert err <= O_TOL[kind], f"{what}: max abs err {err:.3e} > {O_TOL[kind]}"
    assert err <= O_REL[kind] * ref_max + 1e-30, f"{what}: err {err:.3e} vs max|ref| {ref_max:.3e}"
    return err


def check_lse(lse_gpu: torch.Tensor, lse_ref: np.ndarray):
    g = lse_gpu.detach().cpu().numpy().astype(np.float64)
    err = np.abs(g - lse_ref).max()
    assert err <= LSE_TOL, f"lse err {err:.3e}"
    return err


def check_scores(s_gpu: np.ndarray, s_ref: np.ndarray, what: str = "scores"):
    err = np.abs(s_gpu.astype(np.float64) - s_ref)
    bad = err > S_REL * s_ref + 1e-12
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

"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module only draws random numbers and casts them to storage formats; it
contains none of the attention, selection or projection arithmetic.  Both the
HIP path and the CPU oracle consume the bytes it produces (the oracle decodes
them itself from the raw bit patterns).

Recipe (every tensor gets its own torch generator, seeded from the workload
seed and a fixed stream number, so any tensor can be regenerated alone):

* queries, keys and values: N(0, 1) float32 draws scaled by 1/16, cast to the
  storage type (bf16 by round-to-nearest-even; float32 as drawn);
* FP8 caches: the float32 rows above, scaled per row by amax/448, clamped to
  +-448 and cast to OCP e4m3 (round to nearest even); the per-row float32 scale
  is stored next to the codes;
* hidden states of the bridge: N(0, 1); projections: N(0, 0.02^2), both bf16;
* long-prefill "needles": key j is replaced by 8 times the unit vector of the
  head-mean of the (bf16) query of a target token i >= j + 128, so that key j is
  a clear top candidate for query i.

Generation runs on any torch device; large workloads draw directly on the GPU.
"""

from __future__ import annotations

import dataclasses

import numpy as np
import torch

STD_QKV = 1.0 / 16.0
STD_W = 0.02
E4M3_MAX = 448.0

# stream numbers of the per-tensor generators
S_Q, S_K, S_V, S_X, S_WK, S_WV = 0, 1, 2, 3, 4, 5
S_QSPARSE = 100          # + sparse layer number
S_QFULL_LAYER = 1000     # + full layer number (bridge workload)
S_NEEDLES = 7


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "prefill" | "decode" | "bridge" | "swa"
    seed: int
    H: int = 16
    d: int = 256
    B: int = 1
    L: int = 0           # prefill length / bridge rows
    T: int = 0           # decode cache length
    kv: str = "bf16"     # "f32" | "bf16" | "e4m3"
    n_sparse: int = 1    # sparse layers per full layer
    needles: int = 0
    steps: int = 1       # decode steps (consecutive positions at the end of the cache)
    D: int = 0           # bridge hidden size
    n_full: int = 0      # bridged full layers
    window: int = 0      # sliding window (self-decoder SWA layer)
    rope_dims: int = 0   # leading dims turned by the rotary embedding (SWA layer)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_prefill_2k", "prefill", seed=1, H=4, L=2048, kv="f32", n_sparse=1),
        Workload("decode_b16_32k", "decode", seed=2, B=16, T=32768, n_sparse=3),
        Workload("prefill_128k", "prefill", seed=3, L=131072, n_sparse=2, needles=64),
        Workload("bridge_64k", "bridge", seed=4, L=65536, D=2048, n_full=4, n_sparse=8),
        Workload("decode_1m_fp8", "decode", seed=5, T=1 << 20, kv="e4m3", steps=4, n_sparse=4),
        Workload("self_decoder_swa_128k", "swa", seed=6, L=131072, n_sparse=0, window=128, rope_dims=64),
    ]
}


def generator(seed: int, stream: int, device) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed((seed * 1_000_003 + stream) & 0x7FFF_FFFF_FFFF_FFFF)
    return g


def normal(shape, std: float, seed: int, stream: int, device) -> torch.Tensor:
    g = generator(seed, stream, device)
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    return x.mul_(std)


def cast(x: torch.Tensor, kind: str) -> torch.Tensor:
    """float32 -> storage type ("f32" or "bf16")."""
    if kind == "f32":
        return x
    if kind == "bf16":
        return x.to(torch.bfloat16)
    raise ValueError(kind)


def quantize_e4m3_rows(x: torch.Tensor):
    """Per-row FP8 e4m3 codes (uint8) and float32 scales of a float32 tensor."""
    amax = x.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax)).to(torch.float32)
    y = (x / scale.unsqueeze(-1)).clamp_(-E4M3_MAX, E4M3_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.contiguous(), scale.contiguous()


def kv_cache(shape, kind: str, seed: int, device, std: float = STD_QKV):
    """K and V caches of the given shape [..., T, d] in storage type ``kind``.

    Returns (k, v, k_scale, v_scale); the scales are None unless kind == "e4m3".
    """
    kf = normal(shape, std, seed, S_K, device)
    vf = normal(shape, std, seed, S_V, device)
    if kind == "e4m3":
        k, ks = quantize_e4m3_rows(kf)
        v, vs = quantize_e4m3_rows(vf)
        return k, v, ks, vs
    return cast(kf, kind), cast(vf, kind), None, None


def q_dtype_of(kv: str) -> str:
    """Queries are float32 with a float32 cache and bf16 otherwise."""
    return "f32" if kv == "f32" else "bf16"


def attention_inputs(*, B: int, n_q: int, T: int, H: int, d: int, kv: str, n_sparse: int,
                     seed: int, device, std: float = STD_QKV) -> dict:
    """Queries of the full layer and of each sparse layer plus one K/V cache."""
    qk = q_dtype_of(kv)
    k, v, ks, vs = kv_cache((B, T, d), kv, seed, device, std)
    q = cast(normal((B, n_q, H, d), std, seed, S_Q, device), qk)
    qs = [cast(normal((B, n_q, H, d), std, seed, S_QSPARSE + i, device), qk) for i in range(n_sparse)]
    return dict(q=q, k=k, v=v, k_scale=ks, v_scale=vs, q_sparse=qs, kv=kv, q_kind=qk)


def plant_needles(q: torch.Tensor, k: torch.Tensor, n: int, seed: int, window: int = 128):
    """Overwrite ``n`` keys of k [L, d] with needles aimed at later queries of q [L, H, d].

    Needle positions j are drawn without replacement from [0, L-window-1] and
    each gets a target query i uniform in [j+window, L-1].  Returns the list of
    (j, i) pairs.  Works in place on k (same dtype as q).
    """
    L = k.shape[0]
    rng = np.random.default_rng([seed, S_NEEDLES])
    pos = rng.choice(L - window, size=n, replace=False)
    pairs = []
    for j in sorted(int(x) for x in pos):
        i = int(rng.integers(j + window, L))
        m = q[i].to(torch.float32).mean(dim=0)
        k[j] = (8.0 * m / m.norm()).to(k.dtype)
        pairs.append((j, i))
    return pairs


def bridge_inputs(*, L: int, D: int, n_layers: int, d: int, seed: int, device) -> dict:
    x = normal((L, D), 1.0, seed, S_X, device).to(torch.bfloat16)
    wk = normal((n_layers, D, d), STD_W, seed, S_WK, device).to(torch.bfloat16)
    wv = normal((n_layers, D, d), STD_W, seed, S_WV, device).to(torch.bfloat16)
    return dict(x=x, w_k=wk, w_v=wv)


def raw_numpy(t: torch.Tensor | None):
    """Storage bytes of a tensor as a NumPy array the oracle can decode.

    bf16 -> uint16 bit patterns, float32 -> float32, uint8 -> uint8.
    """
    if t is None:
        return None
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype in (torch.float32, torch.uint8, torch.int32):
        return t.numpy()
    raise TypeError(t.dtype)


def kind_of(t: torch.Tensor) -> str:
    return {torch.float32: "f32", torch.bfloat16: "bf16", torch.uint8: "e4m3"}[t.dtype]

"""Plant plausible mistakes in copies of the oracle: the pins must catch each one.

Every mutation below is a one-token slip (an off-by-one bound, a wrong sign,
axis, operand or tie rule).  The mutated source is executed as a throw-away
module on the CPU; the real oracle is untouched.
"""
import os
import sys
import types

import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import oracle_pins  # noqa: E402

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "hs2_oracle.py")

MUTATIONS = [
    ("causal bound off by one", "keys = k[: p + 1]", "keys = k[: p]"),
    ("value rows off by one", "vals = v[: p + 1]", "vals = v[1: p + 2]"),
    ("wrong max sign", "e = np.exp(logits - m)\n        z = e.sum(axis=1, keepdims=True)\n        prob",
     "e = np.exp(logits + m)\n        z = e.sum(axis=1, keepdims=True)\n        prob"),
    ("scale dropped", "logits = sm_scale * (q[i] @ keys.T)", "logits = (q[i] @ keys.T)"),
    ("values used as keys", "logits = sm_scale * (q[i] @ keys.T)", "logits = sm_scale * (q[i] @ vals.T)"),
    ("lse without max", "lse[i] = m[:, 0] + np.log(z[:, 0])\n        scores.append",
     "lse[i] = np.log(z[:, 0])\n        scores.append"),
    ("swa lse without max", "lse[i] = m[:, 0] + np.log(z[:, 0])\n    return o, lse",
     "lse[i] = np.log(z[:, 0])\n    return o, lse"),
    ("score as mean over heads", "scores.append(prob.sum(axis=0))", "scores.append(prob.mean(axis=0))"),
    ("score from first head only", "scores.append(prob.sum(axis=0))", "scores.append(prob[0])"),
    ("unnormalised probabilities", "prob = e / z                            # softmax",
     "prob = e                                # softmax"),
    ("default scale 1/d", "sm_scale = 1.0 / math.sqrt(d)\n    o = np.zeros", "sm_scale = 1.0 / d\n    o = np.zeros"),
    ("tie to higher index", "key=lambda j: (-s[j], j)", "key=lambda j: (-s[j], -j)"),
    ("ascending scores", "key=lambda j: (-s[j], j)", "key=lambda j: (s[j], j)"),
    ("window one short", "n_cand = max(0, n - window)\n    if n_cand <= topk:\n        sel = np.arange", "n_cand = max(0, n - window + 1)\n    if n_cand <= topk:\n        sel = np.arange"),
    ("block window one short", "n_cand = max(0, n - window)\n    if n_cand <= topk:\n        return np.arange", "n_cand = max(0, n - window + 1)\n    if n_cand <= topk:\n        return np.arange"),
    ("window one long", "n_cand = max(0, n - window)\n    if n_cand <= topk:\n        sel = np.arange", "n_cand = max(0, n - window - 1)\n    if n_cand <= topk:\n        sel = np.arange"),
    ("block window one long", "n_cand = max(0, n - window)\n    if n_cand <= topk:\n        return np.arange", "n_cand = max(0, n - window - 1)\n    if n_cand <= topk:\n        return np.arange"),
    ("top-k one short", "top = np.array(order[:topk]", "top = np.array(order[:topk - 1]"),
    ("cut test off by one", "n_cand = max(0, n - window)\n    if n_cand <= topk:\n        sel = np.arange", "n_cand = max(0, n - window)\n    if n_cand < topk:\n        sel = np.arange"),
    ("block cut test off by one", "n_cand = max(0, n - window)\n    if n_cand <= topk:\n        return np.arange", "n_cand = max(0, n - window)\n    if n_cand < topk:\n        return np.arange"),
    ("tau from wrong rank", "tau = float(s[order[topk - 1]])", "tau = float(s[order[topk]])"),
    ("sparse values unsorted", "vals = np.asarray(v, dtype=np.float64)[sel]",
     "vals = np.asarray(v, dtype=np.float64)[np.sort(sel)]"),
    ("sparse scale dropped", "logits = sm_scale * (q @ keys.T)            # [H, |sel|]",
     "logits = (q @ keys.T)            # [H, |sel|]"),
    ("sparse lse sign", "lse = m[:, 0] + np.log(z[:, 0])\n    return o, lse",
     "lse = m[:, 0] - np.log(z[:, 0])\n    return o, lse"),
    ("bridge V from W_k", "v = np.stack([x @ w_v[m]", "v = np.stack([x @ w_k[m]"),
    ("bridge weight rows reversed", "k = np.stack([x @ w_k[m]", "k = np.stack([x @ w_k[m][::-1]"),
    ("bf16 one bit short", "qexp = np.maximum(e - 8, -133)", "qexp = np.maximum(e - 7, -133)"),
    ("bf16 truncation", "r = np.rint(np.ldexp(xf, -qexp))", "r = np.trunc(np.ldexp(xf, -qexp))"),
    ("bf16 decode shift", "<< np.uint32(16)).view", "<< np.uint32(15)).view"),
    ("e4m3 bias 8", "(1.0 + M / 8.0) * 2.0 ** (E - 7)", "(1.0 + M / 8.0) * 2.0 ** (E - 8)"),
    ("e4m3 subnormal step", "t[code] = s * M * 2.0 ** -9", "t[code] = s * M * 2.0 ** -10"),
    ("e4m3 scale ignored", "return vals * np.asarray(scale", "return vals + 0 * np.asarray(scale"),
    ("e4m3 encode truncates", "val = np.rint(a / step) * step", "val = np.floor(a / step) * step"),
    ("e4m3 encode one mantissa bit short", "step = np.ldexp(1.0, ex - 1 - 3)", "step = np.ldexp(1.0, ex - 1 - 2)"),
    ("e4m3 encode sign lost", "np.where(np.signbit(y), 0x80, 0)", "np.where(np.signbit(y), 0, 0)"),
    ("fp8 scale for the fnuz range", "(amax / 448.0).astype(np.float32)", "(amax / 240.0).astype(np.float32)"),
    ("fp8 codes from the reciprocal product", "y = (a / scale[..., None]).astype(np.float32)",
     "y = (a * np.where(amax > 0, (448.0 / np.where(amax > 0, amax, 1.0)).astype(np.float32), 0.0)[..., None])"
     ".astype(np.float32)"),
    ("fp8 quotient in float64", "y = (a / scale[..., None]).astype(np.float32).astype(np.float64)",
     "y = (a / scale[..., None])"),
    ("fp8 V quantized from K", "vc, vs = quantize(v)", "vc, vs = quantize(k)"),
    ("block ties to the higher index", "key=lambda b: (-sig[b], b))", "key=lambda b: (-sig[b], -b))"),
    ("block sums in float32, pairwise tree", "return math.fsum(np.asarray(vals, dtype=np.float64).tolist())",
     "t = np.asarray(vals, dtype=np.float32)\n    while t.size > 1:\n"
     "        t = np.concatenate([t, np.zeros(t.size % 2, np.float32)])\n"
     "        t = (t[0::2] + t[1::2]).astype(np.float32)\n    return float(t[0])"),
    ("block sums in float32, left to right", "return math.fsum(np.asarray(vals, dtype=np.float64).tolist())",
     "return float(np.cumsum(np.asarray(vals, dtype=np.float32), dtype=np.float32)[-1])"),
    ("block sum drops its first token", "return math.fsum(np.asarray(vals, dtype=np.float64).tolist())",
     "return math.fsum(np.asarray(vals, dtype=np.float64)[1:].tolist())"),
    ("block scores its best token", "return math.fsum(np.asarray(vals, dtype=np.float64).tolist())",
     "return float(np.max(vals))"),
    ("block sum counts the window", "sig = [block_score(s[b * block: min(n_cand, (b + 1) * block)])",
     "sig = [block_score(s[b * block: min(n, (b + 1) * block)])"),
    ("block partial block dropped", "nb = (n_cand + block - 1) // block\n    sig", "nb = n_cand // block\n    sig"),
    ("block one block too many", "nsel = topk // block", "nsel = topk // block + 1"),
    ("rope rotation sign", "x[..., 0:rope_dims:2] = even * c - odd * s", "x[..., 0:rope_dims:2] = even * c + odd * s"),
    ("rope pairs are the two halves", "even = x[..., 0:rope_dims:2].copy()\n    odd = x[..., 1:rope_dims:2].copy()",
     "even = x[..., 0:rope_dims // 2].copy()\n    odd = x[..., rope_dims // 2:rope_dims].copy()"),
    ("rope frequency exponent halved", "freq = base ** (-2.0 * m / rope_dims)", "freq = base ** (-m / rope_dims)"),
    ("rope base fixed", "freq = base ** (-2.0 * m / rope_dims)", "freq = 10000.0 ** (-2.0 * m / rope_dims)"),
    ("swa window one long", "lo = max(0, p - window + 1)", "lo = max(0, p - window)"),
    ("swa window one short", "lo = max(0, p - window + 1)", "lo = max(0, p - window + 2)"),
    ("swa keys not rotated", "kr = rope_partial(np.asarray(k, dtype=np.float64)[first: last + 1], "
     "np.arange(first, last + 1), rope_dims, base)", "kr = np.asarray(k, dtype=np.float64)[first: last + 1]"),
    ("swa keys rotated from position 0", "np.arange(first, last + 1), rope_dims, base)",
     "np.arange(0, last + 1 - first), rope_dims, base)"),
    ("swa queries rotated by index", "qpos = q_pos0 + np.arange(n_q)", "qpos = np.arange(n_q)"),
    ("swa values from the rotated keys", "o[i] = (e / z) @ v[lo - first: p + 1 - first]",
     "o[i] = (e / z) @ kr[lo - first: p + 1 - first]"),
    ("block tokens past the candidates", "toks = [np.arange(b * block, min(n_cand, (b + 1) * block)",
     "toks = [np.arange(b * block, min(n, (b + 1) * block)"),
]


def _mutant(old, new):
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation anchor not unique or missing: {old!r}"
    mod = types.ModuleType("hs2_oracle_mutant")
    exec(compile(src.replace(old, new), "hs2_oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_mutation(name, old, new):
    mod = _mutant(old, new)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mod)
        except Exception:  # noqa: BLE001 - any failure counts as caught
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake: {name}"

"""ctypes binding of libhs2 (include/hs2.h): argument marshalling only.

Every function here forwards to the C entry point of the same name; torch is
used for device memory (outputs are allocated with torch.empty when not given)
and for the current stream.  All computation happens in the HIP kernels of
libhs2.so; if the library is missing these functions raise instead of falling
back to anything else.
"""
from __future__ import annotations

import ctypes
import math
import os
import re

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhs2.so")
HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "hs2.h")

HS2_OK, HS2_ERR_NULL, HS2_ERR_SHAPE, HS2_ERR_DTYPE = 0, -1, -2, -3
HS2_ERR_UNSUPPORTED, HS2_ERR_ALIGN, HS2_ERR_WORKSPACE, HS2_ERR_HIP = -4, -5, -6, -7
HS2_F32, HS2_BF16, HS2_FP8E4M3 = 0, 1, 2
HEAD_DIM = 256

_vp, _i, _i64, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_PROTOS = {
    "hs2_full_attn_scored": (_i, [_vp, _i, _i, _i, _i, _i, _vp, _vp, _i, _vp, _vp, _i64, _i64, _f, _vp, _vp, _vp,
                                  _i64, _vp, _sz, _vp]),
    "hs2_full_attn_workspace_bytes": (_sz, [_i, _i, _i, _i64, _i]),
    "hs2_select_topk_window": (_i, [_vp, _i64, _i, _i, _i64, _i64, _i, _i, _vp, _vp, _vp, _sz, _vp]),
    "hs2_select_workspace_bytes": (_sz, [_i, _i, _i64, _i64]),
    "hs2_select_blocks_window": (_i, [_vp, _i64, _i, _i, _i64, _i64, _i, _i, _i, _vp, _vp, _vp, _sz, _vp]),
    "hs2_select_blocks_workspace_bytes": (_sz, [_i, _i, _i64, _i64, _i, _i]),
    "hs2_sparse_attn_reuse": (_i, [_vp, _i, _i, _i, _i, _i, _vp, _vp, _i, _vp, _vp, _i64, _vp, _vp, _i, _f, _vp, _vp,
                                   _vp, _sz, _vp]),
    "hs2_sparse_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "hs2_sparse_attn_reuse_noalloc": (_i, [_vp, _i, _i, _i, _i, _i, _vp, _vp, _i, _vp, _vp, _i64, _vp, _vp, _i, _f,
                                           _vp, _vp, _vp]),
    "hs2_bridge_kv_proj": (_i, [_vp, _i64, _i, _vp, _vp, _i, _i, _vp, _vp, _i64, _vp]),
    "hs2_bridge_kv_proj_fp8": (_i, [_vp, _i64, _i, _vp, _vp, _i, _i, _vp, _vp, _vp, _vp, _i64, _i64, _vp]),
    "hs2_rope_partial": (_i, [_vp, _vp, _i64, _i, _i, _i64, _i, ctypes.c_double, _vp]),
    "hs2_swa_attn": (_i, [_vp, _i, _i, _i, _i, _vp, _vp, _i64, _i64, _i, _f, _vp, _vp, _vp]),
    "hs2_status_str": (ctypes.c_char_p, [_i]),
    "hs2_last_error": (ctypes.c_char_p, []),
    "hs2_version": (_i, []),
}

_lib = None


class Hs2Error(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn} -> {status}: {detail}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libhs2.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m token_level_sparse_full_amd.build`")
        so = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _PROTOS.items():
            fn = getattr(so, name)
            fn.restype, fn.argtypes = res, args
        _lib = so
    return _lib


def header_symbols() -> list[str]:
    """Entry points declared in include/hs2.h."""
    with open(HEADER) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    return sorted(set(re.findall(r"\b(hs2_[a-z0-9_]+)\s*\(", text)))


def check(fn: str, status: int) -> None:
    if status != HS2_OK:
        raise Hs2Error(fn, status, lib().hs2_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dtype_code(t: torch.Tensor) -> int:
    return {torch.float32: HS2_F32, torch.bfloat16: HS2_BF16, torch.uint8: HS2_FP8E4M3}[t.dtype]


def full_attn_workspace_bytes(B: int, n_q: int, H: int, T: int, kv_dtype: int) -> int:
    return int(lib().hs2_full_attn_workspace_bytes(B, n_q, H, T, kv_dtype))


def sparse_workspace_bytes(B: int, n_q: int, H: int, max_sel: int) -> int:
    return int(lib().hs2_sparse_workspace_bytes(B, n_q, H, max_sel))


def workspace(nbytes: int, device) -> torch.Tensor | None:
    """Device scratch of at least nbytes (torch's allocator returns 256-byte aligned blocks)."""
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device) if nbytes > 0 else None


def hs2_full_attn_scored(q, k, v, *, q_pos0: int, sm_scale: float | None = None, k_scale=None, v_scale=None,
                         o=None, lse=None, scores=None, ld_scores: int | None = None, ws=None, stream=None,
                         want_lse: bool = True):
    """Scored full attention.  q [B,n_q,H,256]; k, v [B,T,256]; returns (o, lse, scores)."""
    B, n_q, H, d = q.shape
    T = k.shape[1]
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if ld_scores is None:
        ld_scores = (q_pos0 + n_q + 3) // 4 * 4
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, n_q, H), dtype=torch.float32, device=q.device)
    if scores is None:
        scores = torch.zeros((B, n_q, ld_scores), dtype=torch.float32, device=q.device)
    need = full_attn_workspace_bytes(B, n_q, H, T, _dtype_code(k))
    if ws is None:
        ws = workspace(need, q.device)
    rc = lib().hs2_full_attn_scored(_ptr(q), _dtype_code(q), B, n_q, H, d, _ptr(k), _ptr(v), _dtype_code(k),
                                    _ptr(k_scale), _ptr(v_scale), T, q_pos0, sm_scale, _ptr(o), _ptr(lse),
                                    _ptr(scores), ld_scores, _ptr(ws), 0 if ws is None else ws.numel(),
                                    _stream(stream))
    check("hs2_full_attn_scored", rc)
    return o, lse, scores


def select_workspace_bytes(B: int, n_q: int, T: int, q_pos0: int) -> int:
    return int(lib().hs2_select_workspace_bytes(B, n_q, T, q_pos0))


def hs2_select_topk_window(scores, *, q_pos0: int, T: int, n_q: int | None = None, window: int = 128,
                           topk: int = 1024, idx=None, count=None, ws=None, stream=None):
    """Token-level top-k with forced window.  scores [B,n_q,ld]; returns (idx, count)."""
    B, nq_s, ld = scores.shape
    n_q = nq_s if n_q is None else n_q
    if idx is None:
        idx = torch.empty((B, n_q, window + topk), dtype=torch.int32, device=scores.device)
    if count is None:
        count = torch.empty((B, n_q), dtype=torch.int32, device=scores.device)
    if ws is None:
        ws = workspace(select_workspace_bytes(B, n_q, T, q_pos0), scores.device)
    rc = lib().hs2_select_topk_window(_ptr(scores), ld, B, n_q, T, q_pos0, window, topk, _ptr(idx), _ptr(count),
                                      _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream))
    check("hs2_select_topk_window", rc)
    return idx, count


def hs2_select_blocks_window(scores, *, q_pos0: int, T: int, n_q: int | None = None, window: int = 128,
                             topk: int = 1024, block: int = 64, idx=None, count=None, ws=None, stream=None):
    """Block-level top-k with forced window.  scores [B,n_q,ld]; returns (idx, count) in the
    token-level call's format."""
    B, nq_s, ld = scores.shape
    n_q = nq_s if n_q is None else n_q
    if idx is None:
        idx = torch.empty((B, n_q, window + topk), dtype=torch.int32, device=scores.device)
    if count is None:
        count = torch.empty((B, n_q), dtype=torch.int32, device=scores.device)
    need = int(lib().hs2_select_blocks_workspace_bytes(B, n_q, T, q_pos0, window, block))
    if ws is None:
        ws = workspace(need, scores.device)
    rc = lib().hs2_select_blocks_window(_ptr(scores), ld, B, n_q, T, q_pos0, window, topk, block, _ptr(idx),
                                        _ptr(count), _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream))
    check("hs2_select_blocks_window", rc)
    return idx, count


def select_blocks_workspace_bytes(B: int, n_q: int, T: int, q_pos0: int, window: int = 128, block: int = 64) -> int:
    return int(lib().hs2_select_blocks_workspace_bytes(B, n_q, T, q_pos0, window, block))


def hs2_sparse_attn_reuse(q, k, v, idx, count, *, sm_scale: float | None = None, k_scale=None, v_scale=None,
                          o=None, lse=None, ws=None, stream=None, want_lse: bool = True):
    """Sparse layer over reused indices.  q [B,n_q,H,256]; idx [B,n_q,max_sel]; returns (o, lse)."""
    B, n_q, H, d = q.shape
    T = k.shape[1]
    max_sel = idx.shape[-1]
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, n_q, H), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = workspace(sparse_workspace_bytes(B, n_q, H, max_sel), q.device)
    rc = lib().hs2_sparse_attn_reuse(_ptr(q), _dtype_code(q), B, n_q, H, d, _ptr(k), _ptr(v), _dtype_code(k),
                                     _ptr(k_scale), _ptr(v_scale), T, _ptr(idx), _ptr(count), max_sel, sm_scale,
                                     _ptr(o), _ptr(lse), _ptr(ws), 0 if ws is None else ws.numel(),
                                     _stream(stream))
    check("hs2_sparse_attn_reuse", rc)
    return o, lse


def hs2_sparse_attn_reuse_noalloc(q, k, v, idx, count, *, sm_scale: float | None = None, k_scale=None, v_scale=None,
                                  o=None, lse=None, stream=None, want_lse: bool = True):
    """hs2_sparse_attn_reuse with the library's static scratch instead of a workspace."""
    B, n_q, H, d = q.shape
    T = k.shape[1]
    max_sel = idx.shape[-1]
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, n_q, H), dtype=torch.float32, device=q.device)
    rc = lib().hs2_sparse_attn_reuse_noalloc(_ptr(q), _dtype_code(q), B, n_q, H, d, _ptr(k), _ptr(v),
                                             _dtype_code(k), _ptr(k_scale), _ptr(v_scale), T, _ptr(idx),
                                             _ptr(count), max_sel, sm_scale, _ptr(o), _ptr(lse), _stream(stream))
    check("hs2_sparse_attn_reuse_noalloc", rc)
    return o, lse


def hs2_rope_partial(x, *, pos0: int, rope_dims: int = 64, rope_base: float = 10000.0, out=None, stream=None):
    """Partial rotary embedding of bf16 rows x [n_pos, heads, 256] (or [n_pos, 256]); slot i at position
    pos0 + i.  out=x turns in place; returns the turned rows."""
    n_pos = x.shape[0]
    heads = x.shape[1] if x.dim() == 3 else 1
    d = x.shape[-1]
    if out is None:
        out = torch.empty_like(x)
    rc = lib().hs2_rope_partial(_ptr(x), _ptr(out), n_pos, heads, d, pos0, rope_dims, rope_base, _stream(stream))
    check("hs2_rope_partial", rc)
    return out


def hs2_swa_attn(q, k, v, *, q_pos0: int, window: int = 128, sm_scale: float | None = None, o=None, lse=None,
                 stream=None, want_lse: bool = True):
    """Sliding-window attention on turned queries and keys.  q [B,n_q,H,256] bf16; k, v [B,T,256] bf16;
    returns (o, lse)."""
    B, n_q, H, d = q.shape
    T = k.shape[1]
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, n_q, H), dtype=torch.float32, device=q.device)
    rc = lib().hs2_swa_attn(_ptr(q), B, n_q, H, d, _ptr(k), _ptr(v), T, q_pos0, window, sm_scale, _ptr(o), _ptr(lse),
                            _stream(stream))
    check("hs2_swa_attn", rc)
    return o, lse


def hs2_bridge_kv_proj(x, w_k, w_v, *, k_out=None, v_out=None, out_layer_stride: int | None = None, stream=None):
    """KV Bridging projection.  x [L,D]; w_k, w_v [n_layers,D,256]; returns (k_out, v_out) [n_layers,L,256]."""
    L, D = x.shape
    n_layers, _, d = w_k.shape
    if k_out is None:
        k_out = torch.empty((n_layers, L, d), dtype=torch.bfloat16, device=x.device)
    if v_out is None:
        v_out = torch.empty((n_layers, L, d), dtype=torch.bfloat16, device=x.device)
    if out_layer_stride is None:
        out_layer_stride = k_out.stride(0) if k_out.dim() == 3 else L * d
    rc = lib().hs2_bridge_kv_proj(_ptr(x), L, D, _ptr(w_k), _ptr(w_v), n_layers, d, _ptr(k_out), _ptr(v_out),
                                  out_layer_stride, _stream(stream))
    check("hs2_bridge_kv_proj", rc)
    return k_out, v_out


def hs2_bridge_kv_proj_fp8(x, w_k, w_v, *, k_out=None, v_out=None, k_scale=None, v_scale=None,
                           out_layer_stride: int | None = None, scale_layer_stride: int | None = None, stream=None):
    """KV Bridging projection into an e4m3 cache.  x [L,D]; w_k, w_v [n_layers,D,256];
    returns (k_out, v_out) uint8 codes [n_layers,L,256] and (k_scale, v_scale) float32 [n_layers,L]."""
    L, D = x.shape
    n_layers, _, d = w_k.shape
    if k_out is None:
        k_out = torch.empty((n_layers, L, d), dtype=torch.uint8, device=x.device)
    if v_out is None:
        v_out = torch.empty((n_layers, L, d), dtype=torch.uint8, device=x.device)
    if k_scale is None:
        k_scale = torch.empty((n_layers, L), dtype=torch.float32, device=x.device)
    if v_scale is None:
        v_scale = torch.empty((n_layers, L), dtype=torch.float32, device=x.device)
    if out_layer_stride is None:
        out_layer_stride = k_out.stride(0) if k_out.dim() == 3 else L * d
    if scale_layer_stride is None:
        scale_layer_stride = k_scale.stride(0) if k_scale.dim() == 2 else L
    rc = lib().hs2_bridge_kv_proj_fp8(_ptr(x), L, D, _ptr(w_k), _ptr(w_v), n_layers, d, _ptr(k_out), _ptr(v_out),
                                      _ptr(k_scale), _ptr(v_scale), out_layer_stride, scale_layer_stride,
                                      _stream(stream))
    check("hs2_bridge_kv_proj_fp8", rc)
    return k_out, v_out, k_scale, v_scale

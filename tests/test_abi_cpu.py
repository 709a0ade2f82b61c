"""C-ABI checks that need no GPU: the library loads, exports every entry point
of include/hs2.h, and rejects invalid arguments in host code before any HIP
call (fake device addresses are never dereferenced on these paths)."""
import ctypes

import pytest

from token_level_sparse_full_amd import hs2

A = 0x7F0000000000          # 256-byte aligned fake device address
MIS = A + 8                 # misaligned for 16-byte checks
F32, BF16, FP8 = hs2.HS2_F32, hs2.HS2_BF16, hs2.HS2_FP8E4M3


@pytest.fixture(scope="module")
def lib():
    return hs2.lib()


def test_exports_every_declared_symbol(lib):
    names = hs2.header_symbols()
    assert len(names) == 16
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert lib.hs2_version() == 10100
    for code in range(0, -8, -1):
        assert lib.hs2_status_str(code).decode().startswith("HS2_")
    assert b"unknown" in lib.hs2_status_str(-99)


def full(lib, **kw):
    a = dict(q=A, qd=BF16, B=1, n_q=1, H=16, d=256, k=A, v=A, kvd=BF16, ks=None, vs=None, T=100, q0=99, sc=0.0625,
             o=A, lse=A, scores=A, ld=100, ws=A, wsb=1 << 40)
    a.update(kw)
    return lib.hs2_full_attn_scored(a["q"], a["qd"], a["B"], a["n_q"], a["H"], a["d"], a["k"], a["v"], a["kvd"],
                                    a["ks"], a["vs"], a["T"], a["q0"], a["sc"], a["o"], a["lse"], a["scores"],
                                    a["ld"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), hs2.HS2_ERR_NULL),
    (dict(scores=None), hs2.HS2_ERR_NULL),
    (dict(d=128), hs2.HS2_ERR_UNSUPPORTED),
    (dict(H=3), hs2.HS2_ERR_UNSUPPORTED),
    (dict(H=32), hs2.HS2_ERR_UNSUPPORTED),
    (dict(qd=F32), hs2.HS2_ERR_DTYPE),
    (dict(qd=7), hs2.HS2_ERR_DTYPE),
    (dict(kvd=FP8), hs2.HS2_ERR_NULL),
    (dict(ks=A, vs=A), hs2.HS2_ERR_DTYPE),
    (dict(q=MIS), hs2.HS2_ERR_ALIGN),
    (dict(scores=MIS), hs2.HS2_ERR_ALIGN),
    (dict(q0=100), hs2.HS2_ERR_SHAPE),
    (dict(q0=-1), hs2.HS2_ERR_SHAPE),
    (dict(n_q=0), hs2.HS2_ERR_SHAPE),
    (dict(ld=96), hs2.HS2_ERR_SHAPE),
    (dict(ld=102), hs2.HS2_ERR_SHAPE),
    (dict(sc=0.0), hs2.HS2_ERR_SHAPE),
    (dict(sc=float("nan")), hs2.HS2_ERR_SHAPE),
    (dict(ws=None), hs2.HS2_ERR_WORKSPACE),
    (dict(wsb=16), hs2.HS2_ERR_WORKSPACE),
    (dict(ws=A + 16), hs2.HS2_ERR_ALIGN),
    (dict(kvd=FP8, ks=None, vs=A, n_q=4, q0=96, H=16), hs2.HS2_ERR_NULL),
    (dict(kvd=FP8, ks=A, vs=A + 2, n_q=4, q0=96, H=16), hs2.HS2_ERR_ALIGN),
])
def test_full_attn_rejects(lib, kw, code):
    assert full(lib, **kw) == code
    assert lib.hs2_last_error().decode() != ""


def test_workspace_sizes(lib):
    # decode rows (n_q * H <= 16) need logits and partial states; prefill needs none
    big = lib.hs2_full_attn_workspace_bytes(1, 1, 16, 1 << 20, FP8)
    assert big >= (1 << 20) * 16 * 4
    assert lib.hs2_full_attn_workspace_bytes(1, 2048, 4, 2048, F32) == 0
    assert lib.hs2_full_attn_workspace_bytes(1, 32768, 16, 131072, BF16) >= 32768 * 16 * 4   # lse pass -> P/V pass
    assert lib.hs2_full_attn_workspace_bytes(16, 1, 16, 32768, BF16) >= 16 * 32768 * 16 * 4
    # few long rows (decode) use the multi-workgroup selector: per segment of 4096 candidates
    # a count and up to 512 kept (pattern, index) pairs
    assert lib.hs2_select_workspace_bytes(1, 1, 1 << 20, (1 << 20) - 1) >= (1 << 20) // 4096 * (4 + 512 * 8)
    assert lib.hs2_select_workspace_bytes(16, 1, 32768, 32767) >= 16 * 8 * (4 + 512 * 8)
    assert lib.hs2_select_workspace_bytes(1, 32768, 131072, 98304) == 0     # many rows: one workgroup per row
    assert lib.hs2_select_workspace_bytes(65, 1, 32768, 32767) == 0         # more than 64 rows
    assert lib.hs2_select_workspace_bytes(16, 1, 24000, 23999) == 0         # rows below 24576 candidates
    # few queries (decode) split each selected set into 128-key pieces: per piece max, sum and output
    assert lib.hs2_sparse_workspace_bytes(16, 1, 16, 1152) >= 16 * 9 * 16 * 258 * 4
    assert lib.hs2_sparse_workspace_bytes(1, 64, 16, 1152) > 0
    assert lib.hs2_sparse_workspace_bytes(1, 65, 16, 1152) == 0             # many queries: one workgroup each
    assert lib.hs2_sparse_workspace_bytes(1, 32768, 16, 1152) == 0
    assert lib.hs2_sparse_workspace_bytes(1, 1, 16, 0) == 0


def sel(lib, **kw):
    a = dict(scores=A, ld=1152, B=1, n_q=1, T=1152, q0=1151, w=128, k=1024, idx=A, count=A, ws=None, wsb=0)
    a.update(kw)
    return lib.hs2_select_topk_window(a["scores"], a["ld"], a["B"], a["n_q"], a["T"], a["q0"], a["w"], a["k"],
                                      a["idx"], a["count"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(scores=None), hs2.HS2_ERR_NULL),
    (dict(idx=None), hs2.HS2_ERR_NULL),
    (dict(w=0), hs2.HS2_ERR_SHAPE),
    (dict(k=0), hs2.HS2_ERR_SHAPE),
    (dict(w=2048, k=2049), hs2.HS2_ERR_SHAPE),
    (dict(q0=1152), hs2.HS2_ERR_SHAPE),
    (dict(ld=1150), hs2.HS2_ERR_SHAPE),
    (dict(ld=1153), hs2.HS2_ERR_SHAPE),
    (dict(scores=MIS), hs2.HS2_ERR_ALIGN),
    (dict(idx=A + 2), hs2.HS2_ERR_ALIGN),
    (dict(B=0), hs2.HS2_ERR_SHAPE),
    # one long decode row: the multi-workgroup selector needs a workspace
    (dict(T=70000, ld=70000, q0=69999), hs2.HS2_ERR_WORKSPACE),
    (dict(T=70000, ld=70000, q0=69999, ws=A, wsb=64), hs2.HS2_ERR_WORKSPACE),
    (dict(T=70000, ld=70000, q0=69999, ws=A + 64, wsb=1 << 30), hs2.HS2_ERR_ALIGN),
])
def test_select_rejects(lib, kw, code):
    assert sel(lib, **kw) == code


def sparse(lib, **kw):
    a = dict(q=A, qd=BF16, B=1, n_q=1, H=16, d=256, k=A, v=A, kvd=BF16, ks=None, vs=None, T=100, idx=A, count=A,
             ms=1152, sc=0.0625, o=A, lse=None, ws=A, wsb=1 << 40)
    a.update(kw)
    return lib.hs2_sparse_attn_reuse(a["q"], a["qd"], a["B"], a["n_q"], a["H"], a["d"], a["k"], a["v"], a["kvd"],
                                     a["ks"], a["vs"], a["T"], a["idx"], a["count"], a["ms"], a["sc"], a["o"],
                                     a["lse"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(idx=None), hs2.HS2_ERR_NULL),
    (dict(count=None), hs2.HS2_ERR_NULL),
    (dict(ms=0), hs2.HS2_ERR_SHAPE),
    (dict(ms=5000), hs2.HS2_ERR_SHAPE),
    (dict(d=64), hs2.HS2_ERR_UNSUPPORTED),
    (dict(kvd=FP8), hs2.HS2_ERR_NULL),
    (dict(qd=F32), hs2.HS2_ERR_DTYPE),
    (dict(o=MIS), hs2.HS2_ERR_ALIGN),
    (dict(lse=A + 2), hs2.HS2_ERR_ALIGN),
    (dict(T=0), hs2.HS2_ERR_SHAPE),
    (dict(ws=None), hs2.HS2_ERR_WORKSPACE),
    (dict(wsb=1024), hs2.HS2_ERR_WORKSPACE),
    (dict(ws=A + 16), hs2.HS2_ERR_ALIGN),
])
def test_sparse_rejects(lib, kw, code):
    assert sparse(lib, **kw) == code


def sparse_na(lib, **kw):
    a = dict(q=A, qd=BF16, B=1, n_q=1, H=16, d=256, k=A, v=A, kvd=BF16, ks=None, vs=None, T=100, idx=A, count=A,
             ms=1152, sc=0.0625, o=A, lse=None)
    a.update(kw)
    return lib.hs2_sparse_attn_reuse_noalloc(a["q"], a["qd"], a["B"], a["n_q"], a["H"], a["d"], a["k"], a["v"],
                                             a["kvd"], a["ks"], a["vs"], a["T"], a["idx"], a["count"], a["ms"],
                                             a["sc"], a["o"], a["lse"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(idx=None), hs2.HS2_ERR_NULL),
    (dict(ms=0), hs2.HS2_ERR_SHAPE),
    (dict(d=64), hs2.HS2_ERR_UNSUPPORTED),
    (dict(o=MIS), hs2.HS2_ERR_ALIGN),
    # 64 queries x 17 pieces of 128 keys: more than the 1024 slots of the static scratch
    (dict(B=4, n_q=16, ms=2176), hs2.HS2_ERR_WORKSPACE),
    (dict(B=1, n_q=33, ms=4096), hs2.HS2_ERR_WORKSPACE),
])
def test_sparse_noalloc_rejects(lib, kw, code):
    assert sparse_na(lib, **kw) == code
    assert lib.hs2_last_error().decode() != ""


def bridge(lib, **kw):
    a = dict(x=A, L=4096, D=2048, wk=A, wv=A, n=4, d=256, ko=A, vo=A, st=4096 * 256)
    a.update(kw)
    return lib.hs2_bridge_kv_proj(a["x"], a["L"], a["D"], a["wk"], a["wv"], a["n"], a["d"], a["ko"], a["vo"],
                                  a["st"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), hs2.HS2_ERR_NULL),
    (dict(vo=None), hs2.HS2_ERR_NULL),
    (dict(d=128), hs2.HS2_ERR_UNSUPPORTED),
    (dict(D=2047), hs2.HS2_ERR_SHAPE),
    (dict(D=16), hs2.HS2_ERR_SHAPE),
    (dict(L=0), hs2.HS2_ERR_SHAPE),
    (dict(n=0), hs2.HS2_ERR_SHAPE),
    (dict(n=65), hs2.HS2_ERR_SHAPE),
    (dict(st=4096 * 256 - 1), hs2.HS2_ERR_SHAPE),
    (dict(wk=MIS), hs2.HS2_ERR_ALIGN),
])
def test_bridge_rejects(lib, kw, code):
    assert bridge(lib, **kw) == code


def bridge8(lib, **kw):
    a = dict(x=A, L=4096, D=2048, wk=A, wv=A, n=4, d=256, ko=A, vo=A, ks=A, vs=A, st=4096 * 256, sst=4096)
    a.update(kw)
    return lib.hs2_bridge_kv_proj_fp8(a["x"], a["L"], a["D"], a["wk"], a["wv"], a["n"], a["d"], a["ko"], a["vo"],
                                      a["ks"], a["vs"], a["st"], a["sst"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), hs2.HS2_ERR_NULL),
    (dict(ks=None), hs2.HS2_ERR_NULL),
    (dict(vs=None), hs2.HS2_ERR_NULL),
    (dict(d=128), hs2.HS2_ERR_UNSUPPORTED),
    (dict(D=2047), hs2.HS2_ERR_SHAPE),
    (dict(D=65536 + 32), hs2.HS2_ERR_SHAPE),
    (dict(L=0), hs2.HS2_ERR_SHAPE),
    (dict(n=65), hs2.HS2_ERR_SHAPE),
    (dict(st=4096 * 256 - 1), hs2.HS2_ERR_SHAPE),
    (dict(sst=4095), hs2.HS2_ERR_SHAPE),
    (dict(ko=MIS), hs2.HS2_ERR_ALIGN),
    (dict(ks=A + 2), hs2.HS2_ERR_ALIGN),
])
def test_bridge_fp8_rejects(lib, kw, code):
    assert bridge8(lib, **kw) == code


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(hs2, "_lib", None)
    monkeypatch.setattr(hs2, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        hs2.lib()


def blocks(lib, **kw):
    a = dict(sc=A, ld=2048, B=1, n_q=4, T=2048, q0=2000, w=128, k=1024, blk=64, idx=A, cnt=A, ws=A, wsb=1 << 40)
    a.update(kw)
    return lib.hs2_select_blocks_window(a["sc"], a["ld"], a["B"], a["n_q"], a["T"], a["q0"], a["w"], a["k"],
                                        a["blk"], a["idx"], a["cnt"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(sc=None), hs2.HS2_ERR_NULL),
    (dict(blk=48), hs2.HS2_ERR_UNSUPPORTED),
    (dict(blk=2), hs2.HS2_ERR_UNSUPPORTED),
    (dict(blk=512), hs2.HS2_ERR_UNSUPPORTED),
    (dict(k=1000), hs2.HS2_ERR_SHAPE),
    (dict(w=0), hs2.HS2_ERR_SHAPE),
    (dict(w=128, k=4096), hs2.HS2_ERR_SHAPE),
    (dict(q0=2045), hs2.HS2_ERR_SHAPE),
    (dict(ld=2002), hs2.HS2_ERR_SHAPE),
    (dict(sc=A + 4), hs2.HS2_ERR_ALIGN),
    (dict(ws=None), hs2.HS2_ERR_WORKSPACE),
    (dict(wsb=64), hs2.HS2_ERR_WORKSPACE),
    (dict(ws=A + 16), hs2.HS2_ERR_ALIGN),
    # 16385 candidate blocks of 4 tokens in the last row
    (dict(blk=4, T=65800, ld=65800, q0=65668, n_q=4), hs2.HS2_ERR_UNSUPPORTED),
])
def test_select_blocks_rejects(lib, kw, code):
    assert blocks(lib, **kw) == code
    assert lib.hs2_last_error().decode() != ""


def test_select_blocks_workspace_size(lib):
    # last row p = 2003: 1876 candidates -> 30 blocks of 64, 4 rows of 30 float32 sums
    assert lib.hs2_select_blocks_workspace_bytes(1, 4, 2048, 2000, 128, 64) == 512
    assert lib.hs2_select_blocks_workspace_bytes(1, 4, 2048, 0, 128, 64) == 0
    assert lib.hs2_select_blocks_workspace_bytes(1, 4, 2048, 2000, 128, 48) == 0


def swa(lib, **kw):
    a = dict(q=A, B=1, n_q=4, H=16, d=256, k=A, v=A, T=100, q0=96, w=128, sc=0.0625, o=A, lse=None)
    a.update(kw)
    return lib.hs2_swa_attn(a["q"], a["B"], a["n_q"], a["H"], a["d"], a["k"], a["v"], a["T"], a["q0"], a["w"],
                            a["sc"], a["o"], a["lse"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), hs2.HS2_ERR_NULL),
    (dict(o=None), hs2.HS2_ERR_NULL),
    (dict(d=128), hs2.HS2_ERR_UNSUPPORTED),
    (dict(H=3), hs2.HS2_ERR_UNSUPPORTED),
    (dict(w=0), hs2.HS2_ERR_SHAPE),
    (dict(sc=0.0), hs2.HS2_ERR_SHAPE),
    (dict(q0=97), hs2.HS2_ERR_SHAPE),
    (dict(q0=-1), hs2.HS2_ERR_SHAPE),
    (dict(n_q=0), hs2.HS2_ERR_SHAPE),
    (dict(k=MIS), hs2.HS2_ERR_ALIGN),
    (dict(lse=A + 2), hs2.HS2_ERR_ALIGN),
])
def test_swa_rejects(lib, kw, code):
    assert swa(lib, **kw) == code
    assert lib.hs2_last_error().decode() != ""


def rope(lib, **kw):
    a = dict(x=A, y=A, n=4096, heads=16, d=256, pos0=0, rd=64, base=10000.0)
    a.update(kw)
    return lib.hs2_rope_partial(a["x"], a["y"], a["n"], a["heads"], a["d"], a["pos0"], a["rd"], a["base"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), hs2.HS2_ERR_NULL),
    (dict(d=128), hs2.HS2_ERR_UNSUPPORTED),
    (dict(n=0), hs2.HS2_ERR_SHAPE),
    (dict(heads=0), hs2.HS2_ERR_SHAPE),
    (dict(pos0=-1), hs2.HS2_ERR_SHAPE),
    (dict(pos0=(1 << 40) - 100), hs2.HS2_ERR_SHAPE),
    (dict(rd=12), hs2.HS2_ERR_UNSUPPORTED),
    (dict(rd=264), hs2.HS2_ERR_UNSUPPORTED),
    (dict(base=0.0), hs2.HS2_ERR_SHAPE),
    (dict(base=float("nan")), hs2.HS2_ERR_SHAPE),
    (dict(y=A + 512 * 16), hs2.HS2_ERR_SHAPE),        # overlapping, not equal
    (dict(y=MIS), hs2.HS2_ERR_ALIGN),
])
def test_rope_rejects(lib, kw, code):
    assert rope(lib, **kw) == code
    assert lib.hs2_last_error().decode() != ""

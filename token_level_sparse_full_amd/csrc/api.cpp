// C ABI of libhs2 (declarations and contracts: include/hs2.h).
//
// Every entry point validates its arguments in plain host code first; only
// when all checks pass does it touch HIP (kernel launches on the caller's
// stream).  Errors never enqueue work or write outputs.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/hs2.h"
#include "hs2_internal.hpp"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_last_error[0] = '\0';
  return HS2_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(HS2_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool heads_ok(int H) { return H == 1 || H == 2 || H == 4 || H == 8 || H == 16; }

// 0 <= q_pos0 and q_pos0 + n_q <= T, for n_q >= 1 and 1 <= T <= 2^31 - 1 (no
// sum is formed before its operands are bounded)
bool positions_ok(int64_t q_pos0, int n_q, int64_t T) { return q_pos0 >= 0 && q_pos0 <= T - n_q; }

// B, n_q and T as every entry point requires them (and the workspace queries
// assume): positive, B * n_q and T inside int32
bool rows_ok(int B, int n_q, int64_t T) {
  return B >= 1 && n_q >= 1 && T >= 1 && (int64_t)B * n_q <= 0x7FFFFFFF && T <= 0x7FFFFFFF;
}

constexpr int64_t kMaxBridgeRows = (int64_t)1 << 40;

// (q, kv) dtype pair check shared by the attention entry points.
int check_dtypes(int q_dtype, int kv_dtype, const float* k_scale, const float* v_scale) {
  const bool known = (q_dtype == HS2_F32 || q_dtype == HS2_BF16) &&
                     (kv_dtype == HS2_F32 || kv_dtype == HS2_BF16 || kv_dtype == HS2_FP8E4M3);
  if (!known) return fail(HS2_ERR_DTYPE, "unknown dtype (q=%d, kv=%d)", q_dtype, kv_dtype);
  const bool pair = (q_dtype == HS2_F32 && kv_dtype == HS2_F32) || (q_dtype == HS2_BF16 && kv_dtype == HS2_BF16) ||
                    (q_dtype == HS2_BF16 && kv_dtype == HS2_FP8E4M3);
  if (!pair) return fail(HS2_ERR_DTYPE, "unsupported (q, kv) dtype pair (%d, %d)", q_dtype, kv_dtype);
  if (kv_dtype == HS2_FP8E4M3) {
    if (!k_scale || !v_scale) return fail(HS2_ERR_NULL, "FP8 caches need k_scale and v_scale");
    if (!aligned(k_scale, 4) || !aligned(v_scale, 4)) return fail(HS2_ERR_ALIGN, "scale vectors must be 4-byte aligned");
  } else if (k_scale || v_scale) {
    return fail(HS2_ERR_DTYPE, "k_scale/v_scale are only used with FP8 caches; pass NULL");
  }
  return HS2_OK;
}

int check_attn_common(const void* q, int q_dtype, int B, int n_q, int H, int d, const void* k, const void* v,
                      int kv_dtype, const float* k_scale, const float* v_scale, int64_t T, float sm_scale,
                      const void* o, const float* lse) {
  if (!q || !k || !v || !o) return fail(HS2_ERR_NULL, "q, k, v and o are required");
  if (d != HS2_HEAD_DIM) return fail(HS2_ERR_UNSUPPORTED, "head dim %d unsupported (only %d)", d, HS2_HEAD_DIM);
  if (!heads_ok(H)) return fail(HS2_ERR_UNSUPPORTED, "H=%d unsupported (1, 2, 4, 8 or 16)", H);
  if (B < 1 || n_q < 1 || T < 1) return fail(HS2_ERR_SHAPE, "B, n_q and T must be >= 1 (B=%d n_q=%d T=%lld)", B, n_q, (long long)T);
  if ((int64_t)B * n_q > 0x7FFFFFFF || T > 0x7FFFFFFF) return fail(HS2_ERR_SHAPE, "B*n_q and T must fit in int32");
  if (!(sm_scale > 0.f) || !std::isfinite(sm_scale)) return fail(HS2_ERR_SHAPE, "sm_scale must be finite and > 0");
  const int rc = check_dtypes(q_dtype, kv_dtype, k_scale, v_scale);
  if (rc != HS2_OK) return rc;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
    return fail(HS2_ERR_ALIGN, "q, k, v and o must be 16-byte aligned");
  if (lse && !aligned(lse, 4)) return fail(HS2_ERR_ALIGN, "lse must be 4-byte aligned");
  return HS2_OK;
}

int kv_kind(int dtype) { return dtype == HS2_F32 ? hs2::KV_F32 : (dtype == HS2_BF16 ? hs2::KV_BF16 : hs2::KV_E4M3); }

}  // namespace

extern "C" {

int hs2_version(void) { return 10100; }

const char* hs2_last_error(void) { return g_last_error; }

const char* hs2_status_str(int status) {
  switch (status) {
    case HS2_OK: return "HS2_OK";
    case HS2_ERR_NULL: return "HS2_ERR_NULL: a required pointer is NULL";
    case HS2_ERR_SHAPE: return "HS2_ERR_SHAPE: size out of range or inconsistent";
    case HS2_ERR_DTYPE: return "HS2_ERR_DTYPE: unknown or unsupported dtype";
    case HS2_ERR_UNSUPPORTED: return "HS2_ERR_UNSUPPORTED: configuration not supported";
    case HS2_ERR_ALIGN: return "HS2_ERR_ALIGN: pointer misaligned";
    case HS2_ERR_WORKSPACE: return "HS2_ERR_WORKSPACE: workspace missing or too small";
    case HS2_ERR_HIP: return "HS2_ERR_HIP: HIP launch failed";
    default: return "unknown hs2 status";
  }
}

size_t hs2_full_attn_workspace_bytes(int B, int n_q, int H, int64_t T, int kv_dtype) {
  if (!rows_ok(B, n_q, T) || !heads_ok(H)) return 0;
  return hs2::attn_workspace_bytes(B, n_q, H, T, kv_kind(kv_dtype));
}

int hs2_full_attn_scored(const void* q, int q_dtype, int B, int n_q, int H, int d, const void* k, const void* v,
                         int kv_dtype, const float* k_scale, const float* v_scale, int64_t T, int64_t q_pos0,
                         float sm_scale, void* o, float* lse, float* scores, int64_t ld_scores, void* workspace,
                         size_t ws_bytes, void* stream) {
  int rc = check_attn_common(q, q_dtype, B, n_q, H, d, k, v, kv_dtype, k_scale, v_scale, T, sm_scale, o, lse);
  if (rc != HS2_OK) return rc;
  if (!scores) return fail(HS2_ERR_NULL, "scores is required");
  if (!aligned(scores, 16)) return fail(HS2_ERR_ALIGN, "scores must be 16-byte aligned");
  if (!positions_ok(q_pos0, n_q, T)) return fail(HS2_ERR_SHAPE, "need 0 <= q_pos0 and q_pos0 + n_q <= T");
  if (ld_scores < q_pos0 + n_q || ld_scores % 4 != 0)
    return fail(HS2_ERR_SHAPE, "ld_scores must be >= q_pos0 + n_q and a multiple of 4");
  const size_t need = hs2::attn_workspace_bytes(B, n_q, H, T, kv_kind(kv_dtype));
  if (need > 0) {
    if (!workspace) return fail(HS2_ERR_WORKSPACE, "workspace of %zu bytes required", need);
    if (!aligned(workspace, 256)) return fail(HS2_ERR_ALIGN, "workspace must be 256-byte aligned");
    if (ws_bytes < need) return fail(HS2_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
  }
  hs2::AttnParams p;
  p.q = q; p.k = k; p.v = v; p.k_scale = k_scale; p.v_scale = v_scale;
  p.o = o; p.lse = lse; p.scores = scores; p.ld_scores = ld_scores;
  p.B = B; p.n_q = n_q; p.H = H; p.T = T; p.q_pos0 = q_pos0;
  p.scale_log2 = sm_scale * 1.4426950408889634f;
  return hip_status(hs2::launch_full_attn(p, kv_kind(q_dtype), kv_kind(kv_dtype), workspace, ws_bytes,
                                          (hipStream_t)stream),
                    "hs2_full_attn_scored");
}

size_t hs2_select_workspace_bytes(int B, int n_q, int64_t T, int64_t q_pos0) {
  if (!rows_ok(B, n_q, T) || !positions_ok(q_pos0, n_q, T)) return 0;
  return hs2::select_workspace_bytes(B, n_q, T, q_pos0);
}

int hs2_select_topk_window(const float* scores, int64_t ld_scores, int B, int n_q, int64_t T, int64_t q_pos0,
                           int window, int topk, int32_t* idx, int32_t* count, void* workspace, size_t ws_bytes,
                           void* stream) {
  if (!scores || !idx || !count) return fail(HS2_ERR_NULL, "scores, idx and count are required");
  if (B < 1 || n_q < 1 || T < 1) return fail(HS2_ERR_SHAPE, "B, n_q and T must be >= 1");
  if ((int64_t)B * n_q > 0x7FFFFFFF || T > 0x7FFFFFFF) return fail(HS2_ERR_SHAPE, "B*n_q and T must fit in int32");
  if (window < 1 || topk < 1 || window > HS2_MAX_SELECT || topk > HS2_MAX_SELECT - window)
    return fail(HS2_ERR_SHAPE, "need window >= 1, topk >= 1, window + topk <= %d", HS2_MAX_SELECT);
  if (!positions_ok(q_pos0, n_q, T)) return fail(HS2_ERR_SHAPE, "need 0 <= q_pos0 and q_pos0 + n_q <= T");
  if (ld_scores < q_pos0 + n_q || ld_scores % 4 != 0)
    return fail(HS2_ERR_SHAPE, "ld_scores must be >= q_pos0 + n_q and a multiple of 4");
  if (!aligned(scores, 16)) return fail(HS2_ERR_ALIGN, "scores must be 16-byte aligned");
  if (!aligned(idx, 4) || !aligned(count, 4)) return fail(HS2_ERR_ALIGN, "idx and count must be 4-byte aligned");
  const size_t need = hs2::select_workspace_bytes(B, n_q, T, q_pos0);
  if (need > 0) {
    if (!workspace) return fail(HS2_ERR_WORKSPACE, "workspace of %zu bytes required", need);
    if (!aligned(workspace, 256)) return fail(HS2_ERR_ALIGN, "workspace must be 256-byte aligned");
    if (ws_bytes < need) return fail(HS2_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
  }
  hs2::SelectParams p;
  p.scores = scores; p.ld_scores = ld_scores; p.B = B; p.n_q = n_q; p.q_pos0 = q_pos0;
  p.window = window; p.topk = topk; p.idx = idx; p.count = count;
  return hip_status(hs2::launch_select(p, workspace, ws_bytes, (hipStream_t)stream), "hs2_select_topk_window");
}

static_assert(HS2_MAX_SELECT == hs2::kMaxSelect && HS2_MAX_BLOCKS == hs2::kMaxBlocks, "limits agree");

static bool block_ok(int block) { return block >= 4 && block <= 256 && (block & (block - 1)) == 0; }

size_t hs2_select_blocks_workspace_bytes(int B, int n_q, int64_t T, int64_t q_pos0, int window, int block) {
  if (!rows_ok(B, n_q, T) || !positions_ok(q_pos0, n_q, T) || window < 1 || window > HS2_MAX_SELECT ||
      !block_ok(block))
    return 0;
  return hs2::select_blocks_workspace_bytes(B, n_q, q_pos0, window, block);
}

int hs2_select_blocks_window(const float* scores, int64_t ld_scores, int B, int n_q, int64_t T, int64_t q_pos0,
                             int window, int topk, int block, int32_t* idx, int32_t* count, void* workspace,
                             size_t ws_bytes, void* stream) {
  if (!scores || !idx || !count) return fail(HS2_ERR_NULL, "scores, idx and count are required");
  if (B < 1 || n_q < 1 || T < 1) return fail(HS2_ERR_SHAPE, "B, n_q and T must be >= 1");
  if ((int64_t)B * n_q > 0x7FFFFFFF || T > 0x7FFFFFFF) return fail(HS2_ERR_SHAPE, "B*n_q and T must fit in int32");
  if (window < 1 || topk < 1 || window > HS2_MAX_SELECT || topk > HS2_MAX_SELECT - window)
    return fail(HS2_ERR_SHAPE, "need window >= 1, topk >= 1, window + topk <= %d", HS2_MAX_SELECT);
  if (!block_ok(block)) return fail(HS2_ERR_UNSUPPORTED, "block must be a power of two in [4, 256]");
  if (topk % block != 0) return fail(HS2_ERR_SHAPE, "topk must be a multiple of block");
  if (!positions_ok(q_pos0, n_q, T)) return fail(HS2_ERR_SHAPE, "need 0 <= q_pos0 and q_pos0 + n_q <= T");
  if (ld_scores < q_pos0 + n_q || ld_scores % 4 != 0)
    return fail(HS2_ERR_SHAPE, "ld_scores must be >= q_pos0 + n_q and a multiple of 4");
  if (hs2::select_blocks_nb_max(q_pos0, n_q, window, block) > HS2_MAX_BLOCKS)
    return fail(HS2_ERR_UNSUPPORTED, "more than %d candidate blocks in a row", HS2_MAX_BLOCKS);
  if (!aligned(scores, 16)) return fail(HS2_ERR_ALIGN, "scores must be 16-byte aligned");
  if (!aligned(idx, 4) || !aligned(count, 4)) return fail(HS2_ERR_ALIGN, "idx and count must be 4-byte aligned");
  const size_t need = hs2::select_blocks_workspace_bytes(B, n_q, q_pos0, window, block);
  if (need > 0) {
    if (!workspace) return fail(HS2_ERR_WORKSPACE, "workspace of %zu bytes required", need);
    if (!aligned(workspace, 256)) return fail(HS2_ERR_ALIGN, "workspace must be 256-byte aligned");
    if (ws_bytes < need) return fail(HS2_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
  }
  hs2::SelectParams p;
  p.scores = scores; p.ld_scores = ld_scores; p.B = B; p.n_q = n_q; p.q_pos0 = q_pos0;
  p.window = window; p.topk = topk; p.idx = idx; p.count = count;
  return hip_status(hs2::launch_select_blocks(p, block, workspace, (hipStream_t)stream), "hs2_select_blocks_window");
}

size_t hs2_sparse_workspace_bytes(int B, int n_q, int H, int max_sel) {
  if (!rows_ok(B, n_q, 1) || !heads_ok(H) || max_sel < 1 || max_sel > HS2_MAX_SELECT) return 0;
  return hs2::sparse_workspace_bytes(B, n_q, max_sel);
}

int hs2_sparse_attn_reuse(const void* q, int q_dtype, int B, int n_q, int H, int d, const void* k, const void* v,
                          int kv_dtype, const float* k_scale, const float* v_scale, int64_t T, const int32_t* idx,
                          const int32_t* count, int max_sel, float sm_scale, void* o, float* lse, void* workspace,
                          size_t ws_bytes, void* stream) {
  int rc = check_attn_common(q, q_dtype, B, n_q, H, d, k, v, kv_dtype, k_scale, v_scale, T, sm_scale, o, lse);
  if (rc != HS2_OK) return rc;
  if (!idx || !count) return fail(HS2_ERR_NULL, "idx and count are required");
  if (!aligned(idx, 4) || !aligned(count, 4)) return fail(HS2_ERR_ALIGN, "idx and count must be 4-byte aligned");
  if (max_sel < 1 || max_sel > HS2_MAX_SELECT) return fail(HS2_ERR_SHAPE, "max_sel must be in [1, %d]", HS2_MAX_SELECT);
  const size_t need = hs2::sparse_workspace_bytes(B, n_q, max_sel);
  if (need > 0) {
    if (!workspace) return fail(HS2_ERR_WORKSPACE, "workspace of %zu bytes required", need);
    if (!aligned(workspace, 256)) return fail(HS2_ERR_ALIGN, "workspace must be 256-byte aligned");
    if (ws_bytes < need) return fail(HS2_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
  }
  hs2::SparseParams p;
  p.q = q; p.k = k; p.v = v; p.k_scale = k_scale; p.v_scale = v_scale;
  p.idx = idx; p.count = count; p.o = o; p.lse = lse;
  p.B = B; p.n_q = n_q; p.H = H; p.T = T; p.max_sel = max_sel;
  p.scale_log2 = sm_scale * 1.4426950408889634f;
  return hip_status(hs2::launch_sparse_attn(p, kv_kind(q_dtype), kv_kind(kv_dtype), workspace, (hipStream_t)stream),
                    "hs2_sparse_attn_reuse");
}

int hs2_sparse_attn_reuse_noalloc(const void* q, int q_dtype, int B, int n_q, int H, int d, const void* k,
                                  const void* v, int kv_dtype, const float* k_scale, const float* v_scale, int64_t T,
                                  const int32_t* idx, const int32_t* count, int max_sel, float sm_scale, void* o,
                                  float* lse, void* stream) {
  int rc = check_attn_common(q, q_dtype, B, n_q, H, d, k, v, kv_dtype, k_scale, v_scale, T, sm_scale, o, lse);
  if (rc != HS2_OK) return rc;
  if (!idx || !count) return fail(HS2_ERR_NULL, "idx and count are required");
  if (!aligned(idx, 4) || !aligned(count, 4)) return fail(HS2_ERR_ALIGN, "idx and count must be 4-byte aligned");
  if (max_sel < 1 || max_sel > HS2_MAX_SELECT) return fail(HS2_ERR_SHAPE, "max_sel must be in [1, %d]", HS2_MAX_SELECT);
  const size_t need = hs2::sparse_workspace_bytes(B, n_q, max_sel);
  if (need > hs2::sparse_static_bytes())
    return fail(HS2_ERR_WORKSPACE,
                "%zu bytes of scratch needed, more than the %zu-byte static scratch (B * n_q * ceil(max_sel / 128) "
                "must be at most %d when B * n_q <= 64)",
                need, hs2::sparse_static_bytes(), hs2::kSparseStaticPieces);
  hs2::SparseParams p;
  p.q = q; p.k = k; p.v = v; p.k_scale = k_scale; p.v_scale = v_scale;
  p.idx = idx; p.count = count; p.o = o; p.lse = lse;
  p.B = B; p.n_q = n_q; p.H = H; p.T = T; p.max_sel = max_sel;
  p.scale_log2 = sm_scale * 1.4426950408889634f;
  return hip_status(hs2::launch_sparse_attn_static(p, kv_kind(q_dtype), kv_kind(kv_dtype), (hipStream_t)stream),
                    "hs2_sparse_attn_reuse_noalloc");
}

int hs2_rope_partial(const void* x, void* y, int64_t n_pos, int heads, int d, int64_t pos0, int rope_dims,
                     double rope_base, void* stream) {
  if (!x || !y) return fail(HS2_ERR_NULL, "x and y are required");
  if (d != HS2_HEAD_DIM) return fail(HS2_ERR_UNSUPPORTED, "row width %d unsupported (only %d)", d, HS2_HEAD_DIM);
  constexpr int64_t kMax = (int64_t)1 << 40;
  if (n_pos < 1 || n_pos > kMax || heads < 1 || heads > 4096 || n_pos * heads > kMax)
    return fail(HS2_ERR_SHAPE, "need 1 <= n_pos, 1 <= heads <= 4096, n_pos * heads <= 2^40");
  if (pos0 < 0 || pos0 > kMax - n_pos) return fail(HS2_ERR_SHAPE, "need 0 <= pos0 and pos0 + n_pos <= 2^40");
  if (rope_dims < 0 || rope_dims > HS2_HEAD_DIM || rope_dims % 8 != 0)
    return fail(HS2_ERR_UNSUPPORTED, "rope_dims must be a multiple of 8 in [0, %d]", HS2_HEAD_DIM);
  if (rope_dims > 0 && !(rope_base > 0.0 && std::isfinite(rope_base)))
    return fail(HS2_ERR_SHAPE, "rope_base must be finite and > 0");
  if (!aligned(x, 16) || !aligned(y, 16)) return fail(HS2_ERR_ALIGN, "x and y must be 16-byte aligned");
  const uintptr_t bytes = (uintptr_t)(n_pos * heads) * 512;
  const uintptr_t xa = (uintptr_t)x, ya = (uintptr_t)y;
  if (xa != ya && xa < ya + bytes && ya < xa + bytes)
    return fail(HS2_ERR_SHAPE, "x and y overlap without being equal");
  hs2::RopeParams p{};
  p.x = x; p.y = y; p.n_rows = n_pos * heads; p.heads = heads; p.pos0 = pos0; p.rope_dims = rope_dims;
  return hip_status(hs2::launch_rope(p, rope_base, (hipStream_t)stream), "hs2_rope_partial");
}

int hs2_swa_attn(const void* q, int B, int n_q, int H, int d, const void* k, const void* v, int64_t T, int64_t q_pos0,
                 int window, float sm_scale, void* o, float* lse, void* stream) {
  if (!q || !k || !v || !o) return fail(HS2_ERR_NULL, "q, k, v and o are required");
  if (d != HS2_HEAD_DIM) return fail(HS2_ERR_UNSUPPORTED, "head dim %d unsupported (only %d)", d, HS2_HEAD_DIM);
  if (!heads_ok(H)) return fail(HS2_ERR_UNSUPPORTED, "H=%d unsupported (1, 2, 4, 8 or 16)", H);
  if (!rows_ok(B, n_q, T)) return fail(HS2_ERR_SHAPE, "need B, n_q, T >= 1, B*n_q and T inside int32");
  if (!positions_ok(q_pos0, n_q, T)) return fail(HS2_ERR_SHAPE, "need 0 <= q_pos0 and q_pos0 + n_q <= T");
  if (window < 1) return fail(HS2_ERR_SHAPE, "window must be >= 1");
  if (!(sm_scale > 0.f) || !std::isfinite(sm_scale)) return fail(HS2_ERR_SHAPE, "sm_scale must be finite and > 0");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
    return fail(HS2_ERR_ALIGN, "q, k, v and o must be 16-byte aligned");
  if (lse && !aligned(lse, 4)) return fail(HS2_ERR_ALIGN, "lse must be 4-byte aligned");
  hs2::SwaParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.B = B; p.n_q = n_q; p.H = H; p.T = T; p.q_pos0 = q_pos0; p.window = window;
  p.scale_log2 = sm_scale * 1.4426950408889634f;
  return hip_status(hs2::launch_swa(p, (hipStream_t)stream), "hs2_swa_attn");
}

int hs2_bridge_kv_proj(const void* x, int64_t L, int D, const void* w_k, const void* w_v, int n_layers, int d,
                       void* k_out, void* v_out, int64_t out_layer_stride, void* stream) {
  if (!x || !w_k || !w_v || !k_out || !v_out) return fail(HS2_ERR_NULL, "x, w_k, w_v, k_out and v_out are required");
  if (d != HS2_HEAD_DIM) return fail(HS2_ERR_UNSUPPORTED, "projection width %d unsupported (only %d)", d, HS2_HEAD_DIM);
  if (L < 1 || L > kMaxBridgeRows || D < 32 || D % 32 != 0 || D > 65536)
    return fail(HS2_ERR_SHAPE, "need 1 <= L <= 2^40 and D a multiple of 32 in [32, 65536]");
  if (n_layers < 1 || n_layers > 64) return fail(HS2_ERR_SHAPE, "n_layers must be in [1, 64]");
  if (out_layer_stride < L * (int64_t)d) return fail(HS2_ERR_SHAPE, "out_layer_stride must be >= L * d");
  if ((L + 255) / 256 * (int64_t)(2 * n_layers) > 0x7FFFFFFF) return fail(HS2_ERR_SHAPE, "L too large");
  if (!aligned(x, 16) || !aligned(w_k, 16) || !aligned(w_v, 16) || !aligned(k_out, 16) || !aligned(v_out, 16))
    return fail(HS2_ERR_ALIGN, "x, w_k, w_v, k_out and v_out must be 16-byte aligned");
  hs2::BridgeParams p;
  p.x = x; p.w_k = w_k; p.w_v = w_v; p.k_out = k_out; p.v_out = v_out;
  p.L = L; p.D = D; p.n_layers = n_layers; p.out_layer_stride = out_layer_stride;
  return hip_status(hs2::launch_bridge(p, (hipStream_t)stream), "hs2_bridge_kv_proj");
}

int hs2_bridge_kv_proj_fp8(const void* x, int64_t L, int D, const void* w_k, const void* w_v, int n_layers, int d,
                           uint8_t* k_out, uint8_t* v_out, float* k_scale, float* v_scale, int64_t out_layer_stride,
                           int64_t scale_layer_stride, void* stream) {
  if (!x || !w_k || !w_v || !k_out || !v_out || !k_scale || !v_scale)
    return fail(HS2_ERR_NULL, "x, w_k, w_v, k_out, v_out, k_scale and v_scale are required");
  if (d != HS2_HEAD_DIM) return fail(HS2_ERR_UNSUPPORTED, "projection width %d unsupported (only %d)", d, HS2_HEAD_DIM);
  if (L < 1 || L > kMaxBridgeRows || D < 32 || D % 32 != 0 || D > 65536)
    return fail(HS2_ERR_SHAPE, "need 1 <= L <= 2^40 and D a multiple of 32 in [32, 65536]");
  if (n_layers < 1 || n_layers > 64) return fail(HS2_ERR_SHAPE, "n_layers must be in [1, 64]");
  if (out_layer_stride < L * (int64_t)d) return fail(HS2_ERR_SHAPE, "out_layer_stride must be >= L * d");
  if (scale_layer_stride < L) return fail(HS2_ERR_SHAPE, "scale_layer_stride must be >= L");
  if ((L + 255) / 256 * (int64_t)(2 * n_layers) > 0x7FFFFFFF) return fail(HS2_ERR_SHAPE, "L too large");
  if (!aligned(x, 16) || !aligned(w_k, 16) || !aligned(w_v, 16) || !aligned(k_out, 16) || !aligned(v_out, 16))
    return fail(HS2_ERR_ALIGN, "x, w_k, w_v, k_out and v_out must be 16-byte aligned");
  if (!aligned(k_scale, 4) || !aligned(v_scale, 4)) return fail(HS2_ERR_ALIGN, "k_scale and v_scale must be 4-byte aligned");
  hs2::BridgeParams p;
  p.x = x; p.w_k = w_k; p.w_v = w_v; p.k_out = k_out; p.v_out = v_out;
  p.L = L; p.D = D; p.n_layers = n_layers; p.out_layer_stride = out_layer_stride;
  p.fp8 = true; p.k_scale = k_scale; p.v_scale = v_scale; p.scale_layer_stride = scale_layer_stride;
  return hip_status(hs2::launch_bridge(p, (hipStream_t)stream), "hs2_bridge_kv_proj_fp8");
}

}  // extern "C"

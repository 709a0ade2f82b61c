// Host-side declarations shared between the C-ABI layer (api.cpp) and the
// kernel translation units.  Each launcher enqueues its kernels on `stream`
// and returns the hipError_t of the launch; all arguments have already been
// validated by api.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hs2 {

// storage kinds of K/V (and of Q/O: KV_F32 or KV_BF16)
enum KvKind { KV_F32 = 0, KV_BF16 = 1, KV_E4M3 = 2 };

struct SparseParams {
  const void* q;
  const void* k;
  const void* v;
  const float* k_scale;
  const float* v_scale;
  const int32_t* idx;
  const int32_t* count;
  void* o;
  float* lse;
  int B, n_q, H;
  int64_t T;
  int max_sel;
  float scale_log2;  // sm_scale * log2(e)
};
size_t sparse_workspace_bytes(int B, int n_q, int max_sel);
hipError_t launch_sparse_attn(const SparseParams& p, int q_kind, int kv_kind, void* ws, hipStream_t stream);

// The allocation-free form: the same kernels, with the split form's partial
// states in a static device array of kSparseStaticPieces (query, 128-key piece)
// slots.  Calls whose sparse_workspace_bytes() exceeds sparse_static_bytes()
// must be rejected before the launch.
constexpr int kSparseStaticPieces = 1024;
constexpr size_t sparse_static_bytes() {
  // m and z: 16 floats per piece; o: 16 x 256 floats per piece; each rounded up to 256 B
  return 2 * (((size_t)kSparseStaticPieces * 16 * 4 + 255) & ~(size_t)255) +
         (((size_t)kSparseStaticPieces * 16 * 256 * 4 + 255) & ~(size_t)255);
}
hipError_t launch_sparse_attn_static(const SparseParams& p, int q_kind, int kv_kind, hipStream_t stream);

struct SelectParams {
  const float* scores;
  int64_t ld_scores;
  int B, n_q;
  int64_t q_pos0;
  int window, topk;
  int32_t* idx;
  int32_t* count;
};
size_t select_workspace_bytes(int B, int n_q, int64_t T, int64_t q_pos0);
hipError_t launch_select(const SelectParams& p, void* ws, size_t ws_bytes, hipStream_t stream);

// block-level selection: block in {4, 8, ..., 256}, topk a multiple of block,
// at most kMaxBlocks candidate blocks per row; the workspace holds the block
// sums [B * n_q, nb_max] float32
constexpr int kMaxSelect = 4096;   // largest window + topk
constexpr int kMaxBlocks = 16384;  // candidate blocks of one row held in LDS
int64_t select_blocks_nb_max(int64_t q_pos0, int n_q, int window, int block);
size_t select_blocks_workspace_bytes(int B, int n_q, int64_t q_pos0, int window, int block);
hipError_t launch_select_blocks(const SelectParams& p, int block, void* ws, hipStream_t stream);

struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  const float* k_scale;
  const float* v_scale;
  void* o;
  float* lse;
  float* scores;
  int64_t ld_scores;
  int B, n_q, H;
  int64_t T, q_pos0;
  float scale_log2;
};
bool attn_uses_decode(int n_q, int H);
size_t attn_workspace_bytes(int B, int n_q, int H, int64_t T, int kv_kind);
hipError_t launch_full_attn(const AttnParams& p, int q_kind, int kv_kind, void* ws, size_t ws_bytes,
                            hipStream_t stream);

// self-decoder sliding-window attention (bf16; queries and keys already turned)
struct SwaParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, n_q, H;
  int64_t T, q_pos0;
  int window;
  float scale_log2;        // sm_scale * log2(e)
};
hipError_t launch_swa(const SwaParams& p, hipStream_t stream);

// partial rotary embedding of bf16 rows of 256: row r sits at position
// pos0 + r / heads; x == y turns the leading dims in place
struct RopeParams {
  const void* x;
  void* y;
  int64_t n_rows;
  int heads;
  int64_t pos0;
  int rope_dims;           // a multiple of 8 in [0, 256]
  double rev[128];         // filled by launch_rope: pair m turns rev[m] revolutions per position
};
hipError_t launch_rope(RopeParams p, double rope_base, hipStream_t stream);

struct BridgeParams {
  const void* x;
  const void* w_k;
  const void* w_v;
  void* k_out;
  void* v_out;
  int64_t L;
  int D, n_layers;
  int64_t out_layer_stride;
  // e4m3 output (k_out, v_out hold codes): per-row scales, layer m at m * scale_layer_stride
  bool fp8 = false;
  float* k_scale = nullptr;
  float* v_scale = nullptr;
  int64_t scale_layer_stride = 0;
};
hipError_t launch_bridge(const BridgeParams& p, hipStream_t stream);

}  // namespace hs2

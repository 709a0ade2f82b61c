/*
 * hs2.h - C ABI of the MI355X (gfx950) HySparse2 inner-level attention library.
 *
 * The method (pages on "HySparse2: Hybrid Sparse Attention with Two-Level KV
 * Sharing"): a cross-decoder full-attention layer computes exact causal MQA
 * attention (one K/V head, head dim 256, no positional rotation) and, acting as
 * a selector, scores every past token; each query then keeps the 128 most
 * recent tokens plus the 1024 best-scoring older tokens; the sparse layers that
 * follow attend over those rows of the same K/V cache.  The K/V of the full
 * layer come from KV Bridging: a re-projection of a self-decoder full layer's
 * hidden state with the layer's own projection.
 *
 * Conventions shared by every entry point
 *  - Tensor pointers are DEVICE memory owned by the caller.  The library never
 *    allocates, frees or keeps them beyond the call.  Scratch memory is passed
 *    in as `workspace` (device memory, `ws_bytes` long, 256-byte aligned);
 *    query the size with the matching *_workspace_bytes function.
 *  - Every call enqueues work on `stream` (a hipStream_t passed as void*; NULL
 *    is the null stream) and returns without synchronising.
 *  - Return value: HS2_OK (0) or a negative hs2_status.  All argument checks
 *    are pure host code and run before any HIP call; on an error nothing is
 *    enqueued and no output is written.  HS2_ERR_HIP reports a failed launch;
 *    hs2_last_error() then describes it (thread-local string).
 *  - Layouts are dense, row-major, innermost dimension last.  Pointers must be
 *    16-byte aligned (scale vectors and index/count arrays: 4-byte aligned).
 *  - dtypes: HS2_F32 (float32), HS2_BF16 (bfloat16), HS2_FP8E4M3 (OCP e4m3fn
 *    codes, K/V caches only, each row of 256 codes multiplied by one float32
 *    scale from k_scale / v_scale).  Supported pairs (q, kv): (F32, F32),
 *    (BF16, BF16), (BF16, FP8E4M3).
 *  - Head dim d must be 256; query heads H in {1, 2, 4, 8, 16}.
 *  - Results are deterministic: no floating-point atomics on any output path.
 *  - Inputs are not checked for NaN/Inf; finite results need finite inputs.
 *  - The library is stateless apart from the thread-local error string, and
 *    calls may be made from several host threads.
 */
#ifndef HS2_H_
#define HS2_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum hs2_status {
  HS2_OK = 0,
  HS2_ERR_NULL = -1,        /* a required pointer is NULL                       */
  HS2_ERR_SHAPE = -2,       /* a size is out of range or sizes are inconsistent */
  HS2_ERR_DTYPE = -3,       /* unknown dtype or unsupported (q, kv) pair        */
  HS2_ERR_UNSUPPORTED = -4, /* d != 256, H not in {1,2,4,8,16}, ...             */
  HS2_ERR_ALIGN = -5,       /* a pointer is not aligned as required             */
  HS2_ERR_WORKSPACE = -6,   /* workspace missing or too small                   */
  HS2_ERR_HIP = -7          /* a HIP launch failed; see hs2_last_error()        */
};

enum hs2_dtype { HS2_F32 = 0, HS2_BF16 = 1, HS2_FP8E4M3 = 2 };

#define HS2_HEAD_DIM 256
#define HS2_MAX_HEADS 16
#define HS2_MAX_SELECT 4096 /* largest window + topk accepted by the selector */
#define HS2_MAX_BLOCKS 16384 /* most candidate blocks in one row of the block-level selector */

/*
 * hs2_full_attn_scored - scored full attention (the selector layer).
 *
 * Defines (HySparse2 pages: agihunt.info summary, paragraphs on the inner level
 * and on model shapes -- exact attention scores of the MQA NoPE full layer pick
 * the tokens the sparse layers reuse):
 *   for sequence b, query i at position p = q_pos0 + i, head h:
 *     l_j   = sm_scale * <q[b,i,h,:], k[b,j,:]>           for j = 0..p
 *     P_j   = exp(l_j - lse),  lse = log sum_{j<=p} exp(l_j)
 *     o[b,i,h,:]   = sum_j P_j v[b,j,:]
 *     lse[b,i,h]   = lse
 *     scores[b,i,j] = sum_h P_hj   (probabilities summed over the query heads)
 *
 *   q       [B, n_q, H, d]   q_dtype (HS2_F32 or HS2_BF16)
 *   k, v    [B, T, d]        kv_dtype; for HS2_FP8E4M3 k_scale, v_scale [B, T]
 *                            float32 row scales are required, else they must be NULL
 *   o       [B, n_q, H, d]   written, dtype q_dtype
 *   lse     [B, n_q, H]      float32, natural log; may be NULL
 *   scores  [B, n_q, ld_scores] float32; row i gets columns 0..q_pos0+i, the
 *                            other columns are left untouched
 * Requires 1 <= n_q, 0 <= q_pos0, q_pos0 + n_q <= T, ld_scores >= q_pos0 + n_q,
 * ld_scores a multiple of 4, sm_scale > 0.
 * With an FP8 cache the row scales multiply the logits (k_scale) and the
 * probabilities that weight the V rows (v_scale); the scores are the unscaled
 * probabilities.
 */
int hs2_full_attn_scored(const void* q, int q_dtype, int B, int n_q, int H, int d,
                         const void* k, const void* v, int kv_dtype,
                         const float* k_scale, const float* v_scale, int64_t T,
                         int64_t q_pos0, float sm_scale,
                         void* o, float* lse, float* scores, int64_t ld_scores,
                         void* workspace, size_t ws_bytes, void* stream);

/* Workspace of hs2_full_attn_scored for these shapes:
 *   decode (n_q * H <= 16): float32 logits of every key and row plus the
 *     partial softmax states of the key chunks (about B * T * 64 bytes);
 *   bf16 prefill: the lse of every row in log2 units (B * n_q * H * 4 bytes),
 *     written by the lse pass and read by the probability pass;
 *   FP8 prefill: the same lse, plus the cache widened to bf16 codes
 *     (2 * B * T * 512 bytes: every e4m3 value is exact in bf16), on which the
 *     bf16 kernels then run with the row scales applied per key;
 *   float32 prefill: none (0).
 * The contents are scratch; calls that share a workspace must not overlap. */
size_t hs2_full_attn_workspace_bytes(int B, int n_q, int H, int64_t T, int kv_dtype);

/*
 * hs2_select_topk_window - token-level top-k with the forced recent window.
 *
 * Defines (HySparse2 pages: agihunt.info summary, paragraph on the inner level
 * -- the separate sliding-window branch is removed; the most recent 128 tokens
 * are forced into the selection and the 1024 best-scoring tokens outside that
 * window are added; arXiv abstract -- a sliding window of recent tokens is
 * forced into the sparse selection):
 *   for query i of sequence b at position p = q_pos0 + i:
 *     W = [max(0, p-window+1), p]        (always selected)
 *     C = [0, p-window]                  (candidates)
 *     if |C| <= topk: S = [0, p]
 *     else S = W + the topk candidates of largest score, ties to lower index
 *   idx[b,i,:]  the members of S in ascending order, then -1 up to window+topk
 *   count[b,i]  |S| = min(p+1, window+topk)
 *
 *   scores  [B, n_q, ld_scores] float32, non-negative (as written by
 *           hs2_full_attn_scored); columns 0..p of row i are read
 *   idx     [B, n_q, window+topk] int32, written
 *   count   [B, n_q] int32, written
 * Requires window >= 1, topk >= 1, window + topk <= HS2_MAX_SELECT,
 * q_pos0 + n_q <= T, ld_scores >= q_pos0 + n_q.  The comparison is exact on
 * the float32 values (negative zero, NaN and negative scores are outside the
 * contract).
 */
int hs2_select_topk_window(const float* scores, int64_t ld_scores, int B, int n_q, int64_t T,
                           int64_t q_pos0, int window, int topk,
                           int32_t* idx, int32_t* count,
                           void* workspace, size_t ws_bytes, void* stream);

/* Workspace of hs2_select_topk_window for these shapes (an upper bound over
 * every window >= 1).  It is 0 when the rows are many or short (one workgroup
 * per row); few long rows (at most 64 rows, 24576 or more candidates, the
 * decode case) are split over many workgroups and need, per row, a threshold
 * estimate and, per segment of 4096 candidates, a count and up to 512 kept
 * (score, index) pairs there (about 1 byte per candidate).  The contents are
 * scratch: nothing persists between calls, and calls that share a workspace
 * must not overlap. */
size_t hs2_select_workspace_bytes(int B, int n_q, int64_t T, int64_t q_pos0);

/*
 * hs2_select_blocks_window - block-level top-k with the forced recent window,
 * the granularity that the token-level selection replaces (kept to measure
 * what each costs).
 *
 * Defines (HySparse2 pages: agihunt.info summary, ablation paragraph --
 * token-level against block-level selection at the same 1024-token budget,
 * blocks of 64; 10100.com article, section on the first refinement -- block
 * selection keeps fixed blocks of 64 or 128 tokens).  The pages fix neither
 * the block score nor the window's place; this library takes:
 *   for query i of sequence b at position p = q_pos0 + i:
 *     W = [max(0, p-window+1), p], C = [0, p-window]  (as the token-level call)
 *     if |C| <= topk: S = [0, p]
 *     else: the blocks B_c = [c*block, (c+1)*block - 1] & C, c = 0 .. ceil(|C|/block)-1;
 *           sigma_c = float32 sum of the scores of B_c as a pairwise tree
 *                     (adjacent pairs first, then pairs of those sums, ...);
 *           S = W + the candidates of the topk/block blocks of largest
 *               sigma, ties to the lower block
 *   idx[b,i,:]  the members of S in ascending order, then -1 up to window+topk
 *   count[b,i]  |S| (<= window + topk; less when the last candidate block is
 *               partial and selected)
 *
 *   scores, idx, count as for hs2_select_topk_window; the output feeds
 *   hs2_sparse_attn_reuse unchanged.
 * Requires block a power of two in [4, 256], topk a multiple of block,
 * window >= 1, window + topk <= HS2_MAX_SELECT, at most HS2_MAX_BLOCKS
 * candidate blocks in the last row (ceil((q_pos0 + n_q - window) / block)),
 * and a workspace of hs2_select_blocks_workspace_bytes() bytes (the block
 * sums; scratch, calls sharing it must not overlap).
 */
int hs2_select_blocks_window(const float* scores, int64_t ld_scores, int B, int n_q, int64_t T,
                             int64_t q_pos0, int window, int topk, int block,
                             int32_t* idx, int32_t* count,
                             void* workspace, size_t ws_bytes, void* stream);

/* Workspace of hs2_select_blocks_window: B * n_q * ceil((q_pos0+n_q-window)/block)
 * float32 block sums, rounded up to 256 bytes (0 when no row has candidates;
 * 0 also for invalid arguments). */
size_t hs2_select_blocks_workspace_bytes(int B, int n_q, int64_t T, int64_t q_pos0, int window, int block);

/*
 * hs2_sparse_attn_reuse - a sparse layer over the reused index set.
 *
 * Defines (HySparse2 pages: agihunt.info summary, paragraph on the inner level
 * -- the sparse layers reuse the K/V of the selected tokens, and local and
 * global reads use the same full-attention K/V):
 *   for sequence b, query i, head h, with S = idx[b,i,0..count[b,i]-1]:
 *     o[b,i,h,:] = sum_{j in S} softmax_{j in S}(sm_scale <q[b,i,h,:], k[b,j,:]>) v[b,j,:]
 *     lse[b,i,h] = log sum_{j in S} exp(sm_scale <q[b,i,h,:], k[b,j,:]>)
 *
 *   q      [B, n_q, H, d]    the sparse layer's own queries (q_dtype)
 *   k, v   [B, T, d]         the full layer's cache (kv_dtype, scales as above)
 *   idx    [B, n_q, max_sel] int32 key indices; count [B, n_q] int32
 *   o      [B, n_q, H, d]    written, dtype q_dtype
 *   lse    [B, n_q, H]       float32, may be NULL
 * count is clamped to [0, max_sel]; entries outside [0, T) are skipped (never
 * read).  An empty set yields o = 0 and lse = -inf.  Requires 1 <= max_sel <=
 * HS2_MAX_SELECT, and a workspace of hs2_sparse_workspace_bytes() bytes when
 * that is not 0 (else workspace may be NULL).
 */
int hs2_sparse_attn_reuse(const void* q, int q_dtype, int B, int n_q, int H, int d,
                          const void* k, const void* v, int kv_dtype,
                          const float* k_scale, const float* v_scale, int64_t T,
                          const int32_t* idx, const int32_t* count, int max_sel, float sm_scale,
                          void* o, float* lse, void* workspace, size_t ws_bytes, void* stream);

/* Workspace of hs2_sparse_attn_reuse for these shapes.  It is 0 when the
 * queries are many (B * n_q > 64: one workgroup per query); fewer queries (the
 * decode case) split each selected set into pieces of 128 keys, one workgroup
 * each, and keep every piece's softmax max, sum and unnormalised output there
 * (B * n_q * ceil(max_sel / 128) * 16 * 258 * 4 bytes, rounded up).  The
 * contents are scratch; calls that share a workspace must not overlap.
 * Returns 0 for out-of-range arguments (the call itself then rejects them). */
size_t hs2_sparse_workspace_bytes(int B, int n_q, int H, int max_sel);

/*
 * hs2_sparse_attn_reuse_noalloc - hs2_sparse_attn_reuse for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).
 *
 * Same arguments, results and kernels as hs2_sparse_attn_reuse, without the
 * workspace: the scratch of the split form (B * n_q <= 64) lives in a static
 * device array of the library, 16.9 MB per GPU, held from the first call on a
 * device until the process ends.  It calls no hipMalloc, hipFree or other
 * allocating routine.  Limits: when B * n_q <= 64, B * n_q * ceil(max_sel /
 * 128) must be at most 1024 (e.g. 64 queries with max_sel <= 2048, or 16
 * queries with max_sel <= 4096), else HS2_ERR_WORKSPACE; larger B * n_q need
 * no scratch.  Every call on a GPU shares that GPU's scratch: calls that may
 * overlap on one GPU (several streams, several host threads) race and must
 * be ordered by the caller.  `stream` must belong to the current device.
 */
int hs2_sparse_attn_reuse_noalloc(const void* q, int q_dtype, int B, int n_q, int H, int d,
                                  const void* k, const void* v, int kv_dtype,
                                  const float* k_scale, const float* v_scale, int64_t T,
                                  const int32_t* idx, const int32_t* count, int max_sel, float sm_scale,
                                  void* o, float* lse, void* stream);

/*
 * hs2_rope_partial - rotary position embedding of the leading dims of bf16
 * rows (the embedding of the self-decoder's SWA layers).
 *
 * Defines (HySparse2 pages: agihunt.info summary, model-shapes paragraph --
 * SWA layers use a 64-dim partial RoPE, full and sparse layers none).  The
 * pages give neither the base nor which dims rotate; this library takes the
 * rotary embedding as first defined, on the leading dims: for the row of slot
 * i (position t = pos0 + i) and m < rope_dims / 2,
 *   y[2m]   = x[2m] cos a - x[2m+1] sin a
 *   y[2m+1] = x[2m] sin a + x[2m+1] cos a,     a = t * rope_base^(-2m / rope_dims)
 * and y[j] = x[j] for j >= rope_dims; results rounded to bf16 (RNE).
 *
 *   x, y  [n_pos, heads, d] bf16: every head of slot i sits at position pos0 + i
 *         (heads = H for queries, 1 for K rows).  y == x turns the rows in place
 *         (only the leading rope_dims dims are written); otherwise the two
 *         must not overlap and y receives whole rows.
 * Requires d == 256, n_pos >= 1, 1 <= heads <= 4096, n_pos * heads <= 2^40,
 * pos0 >= 0, pos0 + n_pos <= 2^40, rope_dims a multiple of 8 in [0, 256],
 * rope_base > 0 when rope_dims > 0.  A key is turned once, when it is written
 * to the cache; hs2_swa_attn reads turned rows.
 */
int hs2_rope_partial(const void* x, void* y, int64_t n_pos, int heads, int d, int64_t pos0, int rope_dims,
                     double rope_base, void* stream);

/*
 * hs2_swa_attn - the self-decoder's sliding-window attention (the layers that
 * run before the prefill exits).
 *
 * Defines (HySparse2 pages: agihunt.info summary, backbone paragraph -- the
 * self-decoder mixes full attention with SWA, where each query sees only a
 * recent span of tokens; MQA, head dim 256).  The window length is not given;
 * the window is the `window` most recent keys, the query's own included:
 *   for sequence b, query i at position p = q_pos0 + i, head h:
 *     l_j = sm_scale * <q[b,i,h,:], k[b,j,:]>,  j = max(0, p-window+1) .. p
 *     o[b,i,h,:] = sum_j softmax_j(l) v[b,j,:],  lse[b,i,h] = log sum_j exp(l_j)
 * with queries and keys already turned by hs2_rope_partial (queries at their
 * positions, key j at position j), as the SWA layers use them.
 *
 *   q      [B, n_q, H, d]  bf16;  k, v [B, T, d] bf16
 *   o      [B, n_q, H, d]  bf16, written;  lse [B, n_q, H] float32, may be NULL
 * Requires d == 256, H in {1, 2, 4, 8, 16}, 0 <= q_pos0, q_pos0 + n_q <= T,
 * window >= 1, sm_scale > 0.  No workspace.
 */
int hs2_swa_attn(const void* q, int B, int n_q, int H, int d, const void* k, const void* v, int64_t T,
                 int64_t q_pos0, int window, float sm_scale, void* o, float* lse, void* stream);

/*
 * hs2_bridge_kv_proj - KV Bridging re-projection.
 *
 * Defines (HySparse2 pages: agihunt.info summary, paragraph on the outer level
 * -- a cross-decoder full layer gets its K/V by re-projecting the hidden state
 * of the matching self-decoder full layer, each layer with its own K/V
 * projection; arXiv abstract -- the cross-decoder full-layer KV caches are
 * generated from self-decoder full-layer hidden states):
 *   k_out[m, i, :] = bf16_rne( sum_t x[i,t] * w_k[m,t,:] )   (float32 accumulation)
 *   v_out[m, i, :] = bf16_rne( sum_t x[i,t] * w_v[m,t,:] )
 *
 *   x            [L, D] bf16
 *   w_k, w_v     [n_layers, D, d] bf16
 *   k_out, v_out layer m starts at element m * out_layer_stride; rows of d
 *                elements follow contiguously ([n_layers][L][d] when
 *                out_layer_stride == L*d; a larger stride writes into caches
 *                of T >= L rows, e.g. appending decode rows)
 * Requires L >= 1, D a multiple of 32 in [32, 65536], d == 256,
 * 1 <= n_layers <= 64, out_layer_stride >= L * d, 16-byte aligned x, w_k,
 * w_v, k_out and v_out.  No workspace: the GEMM keeps every partial sum in
 * registers.
 */
int hs2_bridge_kv_proj(const void* x, int64_t L, int D,
                       const void* w_k, const void* w_v, int n_layers, int d,
                       void* k_out, void* v_out, int64_t out_layer_stride, void* stream);

/*
 * hs2_bridge_kv_proj_fp8 - KV Bridging re-projection into an FP8 e4m3 cache.
 *
 * Defines (HySparse2 pages: agihunt.info summary, paragraph on the outer level
 * -- the re-projected K/V fill the cross-decoder caches; same summary, results
 * table and key results -- the KV cache at 1M tokens is counted in FP8): the same
 * projections as hs2_bridge_kv_proj, quantized per output row from the
 * float32 accumulators a[m, i, :] (for k; likewise for v), with amax =
 * max_j |a[m, i, j]| and float32 division:
 *   scale[m, i]    = amax / 448   (1 if the row is 0)
 *   k_out[m, i, j] = e4m3(clamp(a[m, i, j] / scale[m, i], -448, 448))
 * with e4m3 = OCP E4M3 ("e4m3fn") code, round to nearest even, and the
 * quotient the correctly rounded float32 one; the value a code stands for is
 * decode(code) * scale (the cache format hs2_full_attn_scored and
 * hs2_sparse_attn_reuse take with HS2_FP8E4M3, and the one the synthetic
 * inputs use).
 *
 *   x                   [L, D] bf16
 *   w_k, w_v            [n_layers, D, d] bf16
 *   k_out, v_out        uint8 codes; layer m starts at byte m * out_layer_stride,
 *                       rows of d bytes follow contiguously
 *   k_scale, v_scale    float32; layer m starts at element m * scale_layer_stride
 * Requires what hs2_bridge_kv_proj requires, scale_layer_stride >= L, and
 * 4-byte aligned scale pointers.  No workspace.
 */
int hs2_bridge_kv_proj_fp8(const void* x, int64_t L, int D,
                           const void* w_k, const void* w_v, int n_layers, int d,
                           uint8_t* k_out, uint8_t* v_out, float* k_scale, float* v_scale,
                           int64_t out_layer_stride, int64_t scale_layer_stride, void* stream);

/* Human-readable name of a status code (static string). */
const char* hs2_status_str(int status);

/* Detail of the last error on this thread ("" if none). */
const char* hs2_last_error(void);

/* ABI version: major * 10000 + minor * 100 + patch. */
int hs2_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HS2_H_ */

// KV Bridging re-projection.  HySparse2 pages, agihunt.info summary, outer-level
// paragraph: a cross-decoder full layer builds its K/V by re-projecting the
// hidden state of the matching self-decoder full layer with its own K/V
// projection; the arXiv abstract says the cross-decoder full-layer caches are
// generated from self-decoder hidden states.
//
//   k_out[m] = bf16(x W_k[m]),  v_out[m] = bf16(x W_v[m])   (float32 accumulation)
//
// All projections of all bridged layers are one GEMM x[L, D] . [W_k0 | W_v0 |
// W_k1 | ...] with N = 2 * n_layers * 256; the epilogue scatters each 256-wide
// column block to its layer's K or V.  Workgroup tile 256 x 256 (4 waves of
// 128 x 128, 32x32x16 bf16 MFMA), K chunks of 32 staged through LDS and
// prefetched one chunk ahead.  The weights are read in their natural [D][d]
// layout: ds_read_b64_tr_b16 turns the [k][n] LDS tile into the k-contiguous
// B operand, so no transposed copy of W is needed.
#include "hs2_device.hpp"
#include "hs2_internal.hpp"

namespace hs2 {
namespace {

constexpr int BR_THREADS = 256;
constexpr int BM = 256, BN = 256, BK = 32;
constexpr int A_BYTES = BM * BK * 2;  // 16 KB
constexpr int B_BYTES = BK * BN * 2;  // 16 KB

// A tile [BM][BK] bf16: 4 chunks of 16 B per row, chunk ^ ((row >> 2) & 3)
__device__ __forceinline__ int a_off(int row, int ch) { return row * 64 + ((ch ^ ((row >> 2) & 3)) << 4); }
// B tile [BK][BN] bf16: 32 chunks per row, chunk ^ (2 * (row & 3))
__device__ __forceinline__ int b_off(int row, int ch) { return row * 512 + ((ch ^ (2 * (row & 3))) << 4); }

__global__ __launch_bounds__(BR_THREADS, 1) void bridge_kernel(const BridgeParams p) {
  __shared__ __attribute__((aligned(16))) char smem[2 * (A_BYTES + B_BYTES)];
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int hb = l >> 5, l32 = l & 31, G = l >> 4, s16 = l & 15;
  const int wm = wave >> 1, wn = wave & 1;  // wave tile (128 x 128) inside the workgroup tile
  const int n_ntiles = (2 * p.n_layers * 256) / BN;
  const int mt_blk = blockIdx.x / n_ntiles, nt_blk = blockIdx.x % n_ntiles;
  const int64_t m0 = (int64_t)mt_blk * BM;
  const int n0 = nt_blk * BN;                 // global column of the concatenated weights
  const int layer = n0 / 512, which = (n0 / 256) & 1;
  const bf16* x = (const bf16*)p.x;
  const bf16* w = (const bf16*)(which ? p.w_v : p.w_k) + (int64_t)layer * p.D * 256;

  // staging: A 256 rows x 4 chunks, B 32 rows x 32 chunks -> 4 + 4 loads per thread
  auto load = [&](int kc, u32x4* r) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int c = it * BR_THREADS + tid;
      const int row = c >> 2, ch = c & 3;
      const int64_t grow = m0 + row;
      r[it] = grow < p.L ? *(const u32x4*)(x + grow * p.D + kc * BK + ch * 8) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int c = it * BR_THREADS + tid;
      const int row = c >> 5, ch = c & 31;
      r[4 + it] = *(const u32x4*)(w + (int64_t)(kc * BK + row) * 256 + ch * 8);
    }
  };
  auto store = [&](char* buf, const u32x4* r) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int c = it * BR_THREADS + tid;
      *(u32x4*)(buf + a_off(c >> 2, c & 3)) = r[it];
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int c = it * BR_THREADS + tid;
      *(u32x4*)(buf + A_BYTES + b_off(c >> 5, c & 31)) = r[4 + it];
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  const int nk = p.D / BK;
  u32x4 stg[8];
  load(0, stg);
  store(smem, stg);
  __syncthreads();
  for (int kc = 0; kc < nk; ++kc) {
    char* buf = smem + (kc & 1) * (A_BYTES + B_BYTES);
    if (kc + 1 < nk) load(kc + 1, stg);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wm * 128 + 32 * i + l32;
        af[i] = as_bf16x8(*(const u32x4*)(buf + a_off(row, 2 * ks + hb)));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // B[k][n] for k = 16ks + 8(G/2) + i, n = wn*128 + 32j + 16(G%2) + s16
        const int krow = 16 * ks + 8 * (G >> 1) + (s16 >> 2);
        const int col = wn * 128 + 32 * j + 16 * (G & 1) + 4 * (s16 & 3);
        const int ch = col >> 3, half = (col >> 2) & 1;
        const char* b0 = buf + A_BYTES + b_off(krow, ch) + half * 8;
        const char* b1 = buf + A_BYTES + b_off(krow + 4, ch) + half * 8;
        bfr[j] = cat8(lds_tr16((const bf16*)b0), lds_tr16((const bf16*)b1));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
    }
    if (kc + 1 < nk) {
      store(smem + ((kc + 1) & 1) * (A_BYTES + B_BYTES), stg);
      __syncthreads();
    }
  }

  // epilogue: lane holds column wn*128 + 32j + l32, rows wm*128 + 32i + 8(r/4) + 4hb + r%4
  bf16* out = (bf16*)(which ? p.v_out : p.k_out) + (int64_t)layer * p.out_layer_stride;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t grow = m0 + wm * 128 + 32 * i + 8 * (r >> 2) + 4 * hb + (r & 3);
      if (grow >= p.L) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) out[grow * 256 + wn * 128 + 32 * j + l32] = to_bf16(acc[i][j][r]);
    }
}

}  // namespace

size_t bridge_workspace_bytes(int, int, int) { return 0; }

hipError_t launch_bridge(const BridgeParams& p, void*, size_t, hipStream_t stream) {
  const int64_t mtiles = (p.L + BM - 1) / BM;
  const int ntiles = (2 * p.n_layers * 256) / BN;
  hipLaunchKernelGGL(bridge_kernel, dim3((unsigned)(mtiles * ntiles)), dim3(BR_THREADS), 0, stream, p);
  return hipGetLastError();
}

}  // namespace hs2

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
// 128 x 128 in the AGPRs, 32x32x16 bf16 MFMA), K chunks of 32.  The chunks
// stream into LDS by buffer loads to LDS (16 B per lane, no register staging)
// through four stage buffers, three chunks ahead of the MFMAs; each wave's
// eight DMA instructions of a chunk are spread over the 32 MFMAs of the chunk
// before.  The swizzled LDS layouts are made by the per-lane source offsets
// of the DMA.  The weights are read in their natural [D][d] layout:
// ds_read_b64_tr_b16 turns the [k][n] LDS tile into the k-contiguous B
// operand, so no transposed copy of W is needed.  Rows past L read as zeros
// (the buffer resource of the x tile ends at row L).
//
// The e4m3 form (the pages count the KV cache in FP8: agihunt.info summary,
// results table) quantizes each 256-wide output row from its float32
// accumulators: scale = amax / 448 (1 for an all-zero row) and, with
// r = 448 / amax, code = e4m3(clamp(v * r, -448, 448)) rounded to nearest even
// (IEEE float32 division and product; the conversion instruction rounds to
// nearest even): one multiply per element.  A workgroup holds whole rows (its
// 256 columns are one layer's K or V), so the row maxima need only a
// reduction across lanes inside each wave (DPP inside 16-lane rows, then one
// swizzle) and one LDS exchange between the two waves that share a row.
#include "hs2_device.hpp"
#include "hs2_internal.hpp"

namespace hs2 {
namespace {

constexpr int BR_THREADS = 256;
constexpr int BM = 256, BN = 256, BK = 32;
constexpr int A_BYTES = BM * BK * 2;  // 16 KB
constexpr int B_BYTES = BK * BN * 2;  // 16 KB
constexpr int ST_BYTES = A_BYTES + B_BYTES;

// A tile [BM][BK] bf16: 4 chunks of 16 B per row, chunk ^ ((row >> 2) & 3)
__device__ __forceinline__ int a_off(int row, int ch) { return row * 64 + ((ch ^ ((row >> 2) & 3)) << 4); }
// B tile [BK][BN] bf16: 32 chunks per row, chunk ^ (2 * (row & 3))
__device__ __forceinline__ int b_off(int row, int ch) { return row * 512 + ((ch ^ (2 * (row & 3))) << 4); }

// Maximum over the 32 lanes of each half-wave, returned to all of them:
// quad_perm swaps (xor 1, xor 2), the half-row and row mirrors (which pair
// each lane with one in the other half of its 8- and 16-lane group), then one
// swizzle between the two 16-lane rows of the half-wave.
template <int CTRL>
__device__ __forceinline__ float dpp_max(float v) {
  return fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false)));
}
__device__ __forceinline__ float half_wave_max(float v) {
  v = dpp_max<0xB1>(v);    // quad_perm [1,0,3,2]
  v = dpp_max<0x4E>(v);    // quad_perm [2,3,0,1]
  v = dpp_max<0x141>(v);   // row_half_mirror
  v = dpp_max<0x140>(v);   // row_mirror
  return fmaxf(v, shfl_xor(v, 16));
}

template <bool FP8>
__global__ __launch_bounds__(BR_THREADS, 1) void bridge_kernel(const BridgeParams p) {
  // four stage buffers, each its own LDS object so that the compiler can tell
  // the reads of one from the DMA into another
  __shared__ __attribute__((aligned(1024))) char st0[ST_BYTES], st1[ST_BYTES], st2[ST_BYTES], st3[ST_BYTES];
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int hb = l >> 5, l32 = l & 31, G = l >> 4, s16 = l & 15;
  const int wm = wave >> 1, wn = wave & 1;  // wave tile (128 x 128) inside the workgroup tile
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int n_ntiles = (2 * p.n_layers * 256) / BN;
  const int mt_blk = blockIdx.x / n_ntiles, nt_blk = blockIdx.x % n_ntiles;
  const int64_t m0 = (int64_t)mt_blk * BM;
  const int n0 = nt_blk * BN;                 // global column of the concatenated weights
  const int layer = n0 / 512, which = (n0 / 256) & 1;
  const bf16* w = (const bf16*)(which ? p.w_v : p.w_k) + (int64_t)layer * p.D * 256;
  const int nk = p.D / BK;

  // buffer resources: the x rows m0 .. min(L, m0 + 256) - 1 and this weight
  // matrix; empty ones for the chunks past the last (they load zeros, so every
  // chunk issues the same instructions)
  const int rows = (int)min<int64_t>(BM, p.L - m0);
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const bf16*)p.x + m0 * p.D), 0, rows * p.D * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc((void*)w, 0, p.D * 512, 0x00020000);
  const __amdgpu_buffer_rsrc_t r0 = __builtin_amdgcn_make_buffer_rsrc((void*)w, 0, 0, 0x00020000);
  // per-lane source offsets of this wave's DMA instructions i = wv + 4t: LDS
  // chunk 64 i + l holds the source chunk that the swizzle puts there
  uint32_t oa[4], ob[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int P = 64 * (wv + 4 * t) + l;
    const int ar = P >> 2, ach = (P & 3) ^ ((ar >> 2) & 3);
    oa[t] = (uint32_t)(ar * p.D * 2 + ach * 16);
    const int br = P >> 5, bch = (P & 31) ^ (2 * (br & 3));
    ob[t] = (uint32_t)(br * 512 + bch * 16);
  }
  // DMA instruction j (0..7) of chunk kc into stage buffer sb
  auto dma_one = [&](int kc, char* sb, int j) __attribute__((always_inline)) {
    const int t = j & 3, ins = wv + 4 * t;
    const bool live = kc < nk;
    if (j < 4)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(live ? ra : r0, (void HS2_LDS*)((char HS2_LDS*)sb + ins * 1024), 16,
                                               oa[t], kc * (BK * 2), 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(live ? rb : r0, (void HS2_LDS*)((char HS2_LDS*)sb + A_BYTES + ins * 1024),
                                               16, ob[t], kc * (BK * 512), 0, 0);
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  // chunk kc from stage buffer buf; the DMA of chunk kc + 3 into nxt (which
  // held chunk kc - 1) is spread over its MFMAs, one instruction after every
  // fourth
  auto step = [&](int kc, const char* buf, char* nxt) __attribute__((always_inline)) {
    // chunk kc has landed once at most the 16 DMA instructions of the two
    // chunks after it are outstanding; the barrier makes every wave's part
    // visible and ends every wave's reads of chunk kc - 1
    __builtin_amdgcn_s_waitcnt(0x4F70);  // vmcnt(16)
    dma_barrier();
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
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
        dma_one(kc + 3, nxt, 4 * ks + i);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

#pragma unroll
  for (int j = 0; j < 8; ++j) dma_one(0, st0, j);
#pragma unroll
  for (int j = 0; j < 8; ++j) dma_one(1, st1, j);
#pragma unroll
  for (int j = 0; j < 8; ++j) dma_one(2, st2, j);
  for (int kc = 0; kc < nk; kc += 4) {
    step(kc, st0, st3);
    if (kc + 1 < nk) step(kc + 1, st1, st0);
    if (kc + 2 < nk) step(kc + 2, st2, st1);
    if (kc + 3 < nk) step(kc + 3, st3, st2);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the zero-filling DMA past the last chunk

  // epilogue: lane holds column wn*128 + 32j + l32, rows wm*128 + 32i + 8(r/4) + 4hb + r%4
  if constexpr (!FP8) {
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
  } else {
    // row maxima of |v| over this wave's 128 columns (4 per lane, then the 32
    // lanes of the half-wave), then over the partner wave's half through LDS
    float* red = (float*)st0;   // [wm][wn][128 rows]; the DMA has drained
    dma_barrier();              // every wave is done reading the stage buffers
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float m = fmaxf(fmaxf(fabsf(acc[i][0][r]), fabsf(acc[i][1][r])), fmaxf(fabsf(acc[i][2][r]), fabsf(acc[i][3][r])));
        m = half_wave_max(m);
        if (l32 == 0) red[(wm * 2 + wn) * 128 + 32 * i + 8 * (r >> 2) + 4 * hb + (r & 3)] = m;
      }
    dma_barrier();
    uint8_t* out = (uint8_t*)(which ? p.v_out : p.k_out) + (int64_t)layer * p.out_layer_stride;
    float* sc = (which ? p.v_scale : p.k_scale) + (int64_t)layer * p.scale_layer_stride;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * i + 8 * (r >> 2) + 4 * hb + (r & 3);
        const int64_t grow = m0 + wm * 128 + row;
        const float amax = fmaxf(red[(wm * 2) * 128 + row], red[(wm * 2 + 1) * 128 + row]);
        const float scale = amax > 0.f ? amax / 448.f : 1.f;
        const float rcp = amax > 0.f ? 448.f / amax : 0.f;
        if (grow >= p.L) continue;
        if (wn == 0 && l32 == 0) sc[grow] = scale;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float y = __builtin_amdgcn_fmed3f(acc[i][j][r] * rcp, 448.f, -448.f);
          out[grow * 256 + wn * 128 + 32 * j + l32] = (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(y, y, 0, false) & 0xFF);
        }
      }
  }
}

}  // namespace

size_t bridge_workspace_bytes(int, int, int) { return 0; }

hipError_t launch_bridge(const BridgeParams& p, void*, size_t, hipStream_t stream) {
  const int64_t mtiles = (p.L + BM - 1) / BM;
  const int ntiles = (2 * p.n_layers * 256) / BN;
  const dim3 grid((unsigned)(mtiles * ntiles)), block(BR_THREADS);
  if (p.fp8)
    hipLaunchKernelGGL(bridge_kernel<true>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(bridge_kernel<false>, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace hs2

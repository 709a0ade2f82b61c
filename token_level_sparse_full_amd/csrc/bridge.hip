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
// before, and the operand fragments of a chunk's second K-step are read from
// LDS while the MFMAs of its first run.  The tile order gives each XCD a few
// weight blocks for all of its row tiles.  The swizzled LDS layouts are made by the per-lane source offsets
// of the DMA.  The weights are read in their natural [D][d] layout:
// ds_read_b64_tr_b16 turns the [k][n] LDS tile into the k-contiguous B
// operand, so no transposed copy of W is needed.  Rows past L read as zeros
// (the buffer resource of the x tile ends at row L).
//
// The e4m3 form (the pages count the KV cache in FP8: agihunt.info summary,
// results table) quantizes each 256-wide output row from its float32
// accumulators: scale = amax / 448 (1 for an all-zero row) and code =
// e4m3(clamp(v / scale, -448, 448)) rounded to nearest even, with v / scale
// the IEEE float32 quotient.  The quotient costs a multiply and two fma per
// element: with y the correctly rounded 1/scale (one division per row) and
// q0 = v * y, the residual e = fma(-q0, scale, v) is exact and fma(e, y, q0)
// is the correctly rounded v / scale (Markstein's correction step; no
// underflow or overflow arises, |v / scale| <= 448).  The conversion
// instruction rounds to nearest even.  A workgroup holds whole rows (its
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

// Row maxima over the 32 lanes of each half-wave, returned to all of them:
// quad_perm swaps (xor 1, xor 2), the half-row and row mirrors (which pair
// each lane with one in the other half of its 8- and 16-lane group), then one
// swizzle between the two 16-lane rows of the half-wave.  The values are the
// bit patterns of non-negative floats, which order like unsigned integers, so
// integer maxima give the float maximum (and need no NaN quieting between
// the steps, which float maxima of DPP results get).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_umax(uint32_t v) {
  return max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ uint32_t abs_bits(float x) { return __builtin_bit_cast(uint32_t, x) & 0x7fffffffu; }

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
  // Tile order: each XCD (blocks are dealt to the 8 XCDs round-robin) takes a
  // contiguous range of a grouped order -- GN column tiles side by side for
  // every row tile -- so that its L2 holds GN weight blocks (1 MB each) and
  // each x tile is fetched into it once for GN workgroups.
  const int mtiles = (int)(gridDim.x / n_ntiles);
  const int tt = xcd_remap(blockIdx.x, gridDim.x);
  const int GN = n_ntiles % 4 == 0 ? 4 : 2;   // n_ntiles = 2 n_layers is even
  const int grp = tt / (GN * mtiles), rem_t = tt - grp * (GN * mtiles);
  const int mt_blk = rem_t / GN, nt_blk = GN * grp + rem_t % GN;
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

  // Chunk kc from stage buffer buf, its K-step 0 fragments already in
  // registers.  The MFMAs of K-step 0 run while the fragments of K-step 1 are
  // read; then chunk kc + 1 (in nbuf) is waited for, and the barrier sits
  // between the two halves, with the MFMAs of K-step 0 still in flight; the
  // MFMAs of K-step 1 run while the K-step 0 fragments of chunk kc + 1 are
  // read.  So no fragment read waits behind a barrier.  The DMA of chunk kc + 3
  // into nxt (which held chunk kc - 1, whose fragments were all read before
  // the previous step's barrier) is spread over the MFMAs, one instruction
  // after every fourth.
  bf16x8 af[2][4], bfr[2][4];
  auto rd_a = [&](const char* buf, int ks, int i) __attribute__((always_inline)) {
    const int row = wm * 128 + 32 * i + l32;
    return as_bf16x8(*(const u32x4*)(buf + a_off(row, 2 * ks + hb)));
  };
  // B[k][n] for k = 16ks + 8(G/2) + i, n = wn*128 + 32j + 16(G%2) + s16
  auto rd_b = [&](const char* buf, int ks, int j) __attribute__((always_inline)) {
    const int krow = 16 * ks + 8 * (G >> 1) + (s16 >> 2);
    const int col = wn * 128 + 32 * j + 16 * (G & 1) + 4 * (s16 & 3);
    const int ch = col >> 3, half = (col >> 2) & 1;
    const char* b0 = buf + A_BYTES + b_off(krow, ch) + half * 8;
    const char* b1 = buf + A_BYTES + b_off(krow + 4, ch) + half * 8;
    return cat8(lds_tr16((const bf16*)b0), lds_tr16((const bf16*)b1));
  };
  auto step = [&](int kc, const char* buf, const char* nbuf, char* nxt) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(af[0][i], bfr[0][j], acc[i][j]);
      af[1][i] = rd_a(buf, 1, i);
      bfr[1][i] = rd_b(buf, 1, i);
      dma_one(kc + 3, nxt, i);
      __builtin_amdgcn_sched_barrier(0);
    }
    // chunk kc + 1 has landed once at most the 12 DMA instructions issued after
    // it (chunk kc + 2 and the first half of chunk kc + 3) are outstanding
    __builtin_amdgcn_s_waitcnt(0x0F7C);  // vmcnt(12)
    dma_barrier();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(af[1][i], bfr[1][j], acc[i][j]);
      af[0][i] = rd_a(nbuf, 0, i);
      bfr[0][i] = rd_b(nbuf, 0, i);
      dma_one(kc + 3, nxt, 4 + i);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

#pragma unroll
  for (int j = 0; j < 8; ++j) dma_one(0, st0, j);
#pragma unroll
  for (int j = 0; j < 8; ++j) dma_one(1, st1, j);
#pragma unroll
  for (int j = 0; j < 8; ++j) dma_one(2, st2, j);
  // chunk 0 has landed once at most the 16 instructions of chunks 1 and 2 are outstanding
  __builtin_amdgcn_s_waitcnt(0x4F70);  // vmcnt(16)
  dma_barrier();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    af[0][i] = rd_a(st0, 0, i);
    bfr[0][i] = rd_b(st0, 0, i);
  }
  // The main loop runs whole groups of four chunks with no conditions inside:
  // with a conditional step in the body, the compiler could no longer tell
  // which stage buffer each outstanding DMA writes and waited for all but the
  // newest DMA before the first fragment read of a chunk (measured 6 % slower).
  int kc = 0;
  for (; kc + 4 <= nk; kc += 4) {
    step(kc, st0, st1, st3);
    step(kc + 1, st1, st2, st0);
    step(kc + 2, st2, st3, st1);
    step(kc + 3, st3, st0, st2);
  }
  if (kc < nk) {
    step(kc, st0, st1, st3);
    if (kc + 1 < nk) step(kc + 1, st1, st2, st0);
    if (kc + 2 < nk) step(kc + 2, st2, st3, st1);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the zero-filling DMA past the last chunk

  // epilogue: lane holds column wn*128 + 32j + l32, rows wm*128 + 32i + 8(r/4) + 4hb + r%4
  if constexpr (!FP8) {
    bf16* out = (bf16*)(which ? p.v_out : p.k_out) + (int64_t)layer * p.out_layer_stride;
    // the tile's rows m0 .. min(L, m0 + 256) - 1: stores past row L are dropped
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc((void*)(out + m0 * 256), 0, rows * 512, 0x00020000);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 128 + 32 * i + 8 * (r >> 2) + 4 * hb + (r & 3);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, to_bf16(acc[i][j][r])), ro,
                                                (row * 256 + wn * 128 + 32 * j + l32) * 2, 0, 0);
      }
  } else {
    // row maxima of |v| over this wave's 128 columns (4 per lane, then the 32
    // lanes of the half-wave), then over the partner wave's half through LDS
    float* red = (float*)st0;            // [wm][wn][128 rows]; the DMA has drained
    float* rsc = red + 4 * 128;          // [256 rows] scale of each row of the tile
    float* rrc = rsc + 256;              // [256 rows] its correctly rounded reciprocal
    dma_barrier();                       // every wave is done reading the stage buffers
    // eight rows go through each reduction step together, so that no DPP
    // read waits for the write just before it
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r0 = 0; r0 < 16; r0 += 8) {
        uint32_t m[8];
#pragma unroll
        for (int r = 0; r < 8; ++r)
          m[r] = max(max(abs_bits(acc[i][0][r0 + r]), abs_bits(acc[i][1][r0 + r])),
                     max(abs_bits(acc[i][2][r0 + r]), abs_bits(acc[i][3][r0 + r])));
#pragma unroll
        for (int r = 0; r < 8; ++r) m[r] = dpp_umax<0xB1>(m[r]);    // quad_perm [1,0,3,2]
#pragma unroll
        for (int r = 0; r < 8; ++r) m[r] = dpp_umax<0x4E>(m[r]);    // quad_perm [2,3,0,1]
#pragma unroll
        for (int r = 0; r < 8; ++r) m[r] = dpp_umax<0x141>(m[r]);   // row_half_mirror
#pragma unroll
        for (int r = 0; r < 8; ++r) m[r] = dpp_umax<0x140>(m[r]);   // row_mirror
#pragma unroll
        for (int r = 0; r < 8; ++r) m[r] = max(m[r], (uint32_t)__shfl_xor((int)m[r], 16, kWave));
        if (l32 == 0) {
#pragma unroll
          for (int r = 0; r < 8; ++r)
            red[(wm * 2 + wn) * 128 + 32 * i + 8 * ((r0 + r) >> 2) + 4 * hb + ((r0 + r) & 3)] = __builtin_bit_cast(float, m[r]);
        }
      }
    dma_barrier();
    // one thread per row of the tile: the scale (and its reciprocal) is
    // computed once, not by every lane that holds part of the row
    float* sc = (which ? p.v_scale : p.k_scale) + (int64_t)layer * p.scale_layer_stride;
    {
      const int row = tid, rw = row >> 7, rr = row & 127;
      const float amax = fmaxf(red[(rw * 2) * 128 + rr], red[(rw * 2 + 1) * 128 + rr]);
      const float scale = amax > 0.f ? amax / 448.f : 1.f;
      rsc[row] = scale;
      rrc[row] = 1.f / scale;
      if (m0 + row < p.L) sc[m0 + row] = scale;
    }
    dma_barrier();
    uint8_t* out = (uint8_t*)(which ? p.v_out : p.k_out) + (int64_t)layer * p.out_layer_stride;
    // the tile's rows m0 .. min(L, m0 + 256) - 1: stores past row L are dropped
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc((void*)(out + m0 * 256), 0, rows * 256, 0x00020000);
    // A lane holds the codes of columns 32j + l32 (j = 0..3) of a row; a 4 x 4
    // byte transpose inside each quad of lanes (two DPP swaps and two byte
    // permutes) gives lane 4a + t the codes of columns 32t + 4a .. +3, stored
    // as one dword: a half-wave writes a row's 128 codes as one 128-byte line.
    const int qt = l32 & 3;
    // byte selectors of __builtin_amdgcn_perm(hi, lo, sel): bytes 0-3 of lo are
    // 0-3, bytes of hi are 4-7; the first byte of the result is sel's low byte
    const uint32_t sel1 = (qt & 1) ? 0x03070105u : 0x06020400u;   // odd: {X.b1, D.b1, X.b3, D.b3}
    const uint32_t sel2 = (qt & 2) ? 0x03020706u : 0x05040100u;   // lanes 2, 3: {Y.b2, Y.b3, A.b2, A.b3}
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * i + 8 * (r >> 2) + 4 * hb + (r & 3);
        const float scale = rsc[wm * 128 + row], rcp = rrc[wm * 128 + row];
        float y[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float a = acc[i][j][r];
          const float q0 = a * rcp;
          const float q = __builtin_fmaf(__builtin_fmaf(-q0, scale, a), rcp, q0);  // fl32(a / scale)
          y[j] = __builtin_amdgcn_fmed3f(q, 448.f, -448.f);
        }
        int d = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);   // bytes 0, 1: j = 0, 1
        d = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], d, true);        // bytes 2, 3: j = 2, 3
        const int x = __builtin_amdgcn_mov_dpp(d, 0xB1, 0xf, 0xf, false);   // quad_perm [1,0,3,2]
        const int aa = (int)__builtin_amdgcn_perm((uint32_t)x, (uint32_t)d, sel1);
        const int yy = __builtin_amdgcn_mov_dpp(aa, 0x4E, 0xf, 0xf, false); // quad_perm [2,3,0,1]
        const int bb = (int)__builtin_amdgcn_perm((uint32_t)yy, (uint32_t)aa, sel2);
        __builtin_amdgcn_raw_buffer_store_b32((uint32_t)bb, ro, (wm * 128 + row) * 256 + wn * 128 + 32 * qt + 4 * (l32 >> 2),
                                              0, 0);
      }
  }
}

}  // namespace

hipError_t launch_bridge(const BridgeParams& p, hipStream_t stream) {
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

// Self-decoder sliding-window attention and partial rotary embedding.
// HySparse2 pages, agihunt.info summary: the self-decoder mixes full attention
// with sliding-window attention (each query sees only a recent span of
// tokens); the SWA layers use a 64-dim partial RoPE, while the full and sparse
// layers use none; one K/V head (MQA), head dim 256.  These are the attention
// layers that run before the prefill exits at the self-decoder.
//
//   rope(x, t): the pair (x[2m], x[2m+1]), m < rope_dims / 2, turned by the
//               angle t * base^(-2m / rope_dims) (t: the row's position)
//   swa:        o_h = sum_{j = max(0, p-W+1)}^{p} softmax_j(scale <q'_h, k'_j>) v_j
//               on queries and keys already turned by rope
//
// As in a serving cache, a key row is turned once, when it is written
// (rope_kernel), and the attention reads the turned rows.
//
// rope_kernel: one thread per 16-byte chunk (8 dims, 4 pairs) of the turned
// dims.  The angle (position times the pair's frequency in revolutions) is
// formed and reduced in float64 -- positions reach 2^20, where a float32
// product would be off by a tenth of a radian -- and v_sin_f32 / v_cos_f32
// take the fraction of a revolution.
//
// swa_kernel: one sweep with an online softmax over 32-key tiles.
//  * Workgroup: 4 waves x 32 rows (32/H tokens x H heads per wave); the tiles
//    cover the workgroup's key span [first position - W + 1, last position].
//    Consecutive token blocks go to the same XCD, so the tiles they share are
//    fetched into one L2.
//  * K and V tiles stream into LDS by buffer loads to LDS (16 B per lane, no
//    register staging), one tile ahead, into padded rows; the buffer
//    resource of a tile ends at the workgroup's last key, so rows past it
//    read as zeros.
//  * S^T = K Q^T with 32x32x16 bf16 MFMAs: a lane owns one query row and 16
//    keys of the tile, so the row max and sum are in-lane plus one swap with
//    the lane 32 away.
//  * O^T += V^T P^T: P goes from registers straight into the B operand; the
//    contraction order of the keys is permuted to match the registers (lane
//    half hb holds keys 4hb..4hb+3 and 8+4hb..8+4hb+3 of each 16), and the
//    transposed LDS reads of V (ds_read_b64_tr_b16) deliver the same order.
//    A lane also owns its row of O^T, so the rescale is lane-local.
#include <cmath>

#include "hs2_device.hpp"
#include "hs2_internal.hpp"

namespace hs2 {
namespace {

constexpr int SW_WAVES = 4;
constexpr int SW_THREADS = SW_WAVES * kWave;
constexpr int SW_KT = 32;                    // keys per tile
constexpr int SW_KC = 33, SW_VC = 34;        // 16-byte chunks per padded K / V row in LDS
constexpr int SW_KP = SW_KC * 16;            // K row pitch: 16 rows at one chunk hit distinct banks
constexpr int SW_VP = SW_VC * 16;            // V row pitch: the transposed reads hit distinct banks
constexpr int SW_TILE = 17 * 1024;           // one padded tile image (32 x 34 chunks fits 17 DMA instructions)

// ---------------------------------------------------------------- rope
template <bool INPLACE>
__global__ __launch_bounds__(256) void rope_kernel(const RopeParams p) {
  const int cpr = INPLACE ? p.rope_dims / 8 : 32;      // chunks handled per row
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = c / cpr;
  const int ch = (int)(c % cpr);
  if (row >= p.n_rows) return;
  const int64_t pos = p.pos0 + row / p.heads;
  const u32x4 raw = *(const u32x4*)((const char*)p.x + row * 512 + ch * 16);
  u32x4 out = raw;
  if (8 * ch < p.rope_dims) {
    bf16x8 v = as_bf16x8(raw);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const double r = (double)pos * p.rev[4 * ch + i];
      const float t = (float)(r - __builtin_floor(r));   // fraction of a revolution, [0, 1)
      const float cs = __builtin_amdgcn_cosf(t), sn = __builtin_amdgcn_sinf(t);
      const float x0 = (float)v[2 * i], x1 = (float)v[2 * i + 1];
      v[2 * i] = to_bf16(x0 * cs - x1 * sn);
      v[2 * i + 1] = to_bf16(x0 * sn + x1 * cs);
    }
    out = as_u32x4(v);
  }
  *(u32x4*)((char*)p.y + row * 512 + ch * 16) = out;
}

// ---------------------------------------------------------------- swa
template <int H>
__global__ __launch_bounds__(SW_THREADS, 2) void swa_kernel(const SwaParams p) {
  constexpr int TPW = 32 / H;           // tokens per wave
  constexpr int TPB = SW_WAVES * TPW;   // tokens per workgroup
  __shared__ __attribute__((aligned(1024))) char lds_k0[SW_TILE], lds_k1[SW_TILE];
  __shared__ __attribute__((aligned(1024))) char lds_v0[SW_TILE], lds_v1[SW_TILE];

  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int hb = l >> 5, l32 = l & 31, G = l >> 4, s16 = l & 15;
  // neighbouring token blocks share most key tiles: give each XCD (and its L2)
  // a contiguous range of them
  const int blk = xcd_remap(blockIdx.x, gridDim.x);
  const int nblk_tok = (p.n_q + TPB - 1) / TPB;
  const int b = blk / nblk_tok;
  const int tok_blk0 = (blk % nblk_tok) * TPB;
  const int tok = tok_blk0 + wave * TPW + l32 / H;   // this lane's row: token tok, head l32 % H
  const bool row_ok = tok < p.n_q;
  const int64_t my_pos = p.q_pos0 + (row_ok ? tok : p.n_q - 1);
  const int64_t lo_pos = my_pos - p.window + 1;      // oldest key of the row's window (may be < 0)
  const int64_t pos_first = p.q_pos0 + tok_blk0;
  const int64_t n_keys = p.q_pos0 + min(tok_blk0 + TPB, p.n_q);   // keys 0 .. n_keys - 1 exist for the block
  const int64_t kbeg = max((int64_t)0, pos_first - p.window + 1);
  const int kt0 = (int)(kbeg / SW_KT), kt1 = (int)((n_keys - 1) / SW_KT);
  const int64_t q_row = ((int64_t)b * p.n_q + (row_ok ? tok : p.n_q - 1)) * H + (l32 % H);
  const char* kg = (const char*)p.k + (int64_t)b * p.T * 512;
  const char* vg = (const char*)p.v + (int64_t)b * p.T * 512;

  // The wave's 32 rows (32/H tokens x H heads) are one contiguous 16 KB run of
  // q and of o: both move in whole rows, so that every global access
  // instruction covers 1 KB of consecutive bytes, and LDS turns them to and
  // from the MFMA layout (a row per lane).  Read or written in that layout,
  // each instruction would touch 32 rows and issue 32 partial-line requests.
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int tok_w0 = tok_blk0 + wv * TPW;
  const int64_t row_w0 = ((int64_t)b * p.n_q + tok_w0) * H;          // first row of the wave
  const int rows_w = max(0, min(TPW, p.n_q - tok_w0)) * H;             // rows of real tokens
  char* const wbuf = wv == 0 ? lds_k1 : wv == 1 ? lds_v1 : wv == 2 ? lds_k0 : lds_v0;   // the wave's O staging
  // buffer resources over the wave's rows of q and o: loads past the last
  // token return zeros, stores there are dropped
  auto rows_rsrc = [&](const void* base) __attribute__((always_inline)) {
    const uint64_t a = (uint64_t)((const char*)base + row_w0 * 512);
    return __builtin_amdgcn_make_buffer_rsrc(
        (void*)(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) << 32) |
                (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a)),
        0, __builtin_amdgcn_readfirstlane(rows_w * 512), 0x00020000);
  };
  const __amdgpu_buffer_rsrc_t rqo_q = rows_rsrc(p.q);

  uint32_t koff[5], voff[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int c = 64 * (wv + 4 * i) + l;
    const int kr = c / SW_KC, kc = c - kr * SW_KC;
    const int vr = c / SW_VC, vc = c - vr * SW_VC;
    koff[i] = (uint32_t)(min(kr, SW_KT - 1) * 512 + (kc < 32 ? kc : 0) * 16);
    voff[i] = (uint32_t)(min(vr, SW_KT - 1) * 512 + (vc < 32 ? vc : 0) * 16);
  }
  auto dma = [&](int kt, char* kb, char* vb) __attribute__((always_inline)) {
    const int64_t rows = max((int64_t)0, min((int64_t)SW_KT, n_keys - (int64_t)kt * SW_KT));
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void*)(kg + (int64_t)kt * (SW_KT * 512)), 0, (int)(rows * 512), 0x00020000);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc((void*)(vg + (int64_t)kt * (SW_KT * 512)), 0, (int)(rows * 512), 0x00020000);
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const int ins = wv + 4 * i;
      if (i < 4 || wv == 0) {   // 17 instructions per image: wave 0 issues the last one
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (void HS2_LDS*)((char HS2_LDS*)kb + ins * 1024), 16, koff[i], 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (void HS2_LDS*)((char HS2_LDS*)vb + ins * 1024), 16, voff[i], 0, 0, 0);
      }
    }
  };

  // ---- queries (B operand of S^T): row l32, dims 16 s + 8 hb .. +7.  Loaded
  // as whole rows (instruction j: rows 2j and 2j + 1, rows past the last token
  // as zeros) while the first tile's DMA is in flight, then turned into
  // fragments through LDS: in the two buffers of the second tile, waves 0 and
  // 1 first, then waves 2 and 3.
  bf16x8 qf[16];
  {
    u32x4 raw[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
      raw[j] = __builtin_amdgcn_raw_buffer_load_b128(rqo_q, (2 * j + hb) * 512 + 16 * l32, 0, 0);
    dma(kt0, lds_k0, lds_v0);
    auto stage = [&](char* sb) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < 16; ++j) *(u32x4*)(sb + (2 * j + hb) * SW_KP + 16 * l32) = raw[j];
#pragma unroll
      for (int s = 0; s < 16; ++s) qf[s] = as_bf16x8(*(const u32x4*)(sb + l32 * SW_KP + (2 * s + hb) * 16));
    };
    if (wv < 2) stage(wv == 0 ? lds_k1 : lds_v1);
    __syncthreads();
    if (wv >= 2) stage(wv == 2 ? lds_k1 : lds_v1);
  }

  float m_run = kNegInf, z_run = 0.f;
  f32x16 oacc[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) oacc[n] = f32x16{};

  // operands are read SW_AHEAD MFMA steps ahead of their use, and the steps are
  // kept in order, so that only a few fragments are live next to Q and O
  constexpr int SW_AHEAD = 2;
  auto step = [&](int kt, const char* kb, const char* vb) __attribute__((always_inline)) {
    // S^T = K Q^T: lane l holds keys 8(r/4) + 4hb + r%4 of the tile for row l32
    f32x16 st = f32x16{};
    {
      auto kfrag = [&](int s) { return as_bf16x8(*(const u32x4*)(kb + l32 * SW_KP + (2 * s + hb) * 16)); };
      bf16x8 kf[16];
#pragma unroll
      for (int s = 0; s < SW_AHEAD; ++s) kf[s] = kfrag(s);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        st = mfma32(kf[s], qf[s], st);
        if (s + SW_AHEAD < 16) kf[s + SW_AHEAD] = kfrag(s + SW_AHEAD);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // the row's window relative to the tile's first key, as small ints
    const int64_t kbase = (int64_t)kt * SW_KT;
    const int rel_lo = (int)max((int64_t)-1, min((int64_t)SW_KT, lo_pos - kbase));
    const int rel_hi = row_ok ? (int)max((int64_t)-1, min((int64_t)SW_KT, my_pos - kbase)) : -1;
    float x[16];
    float tmax = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 8 * (r >> 2) + 4 * hb + (r & 3);
      const bool ok = key >= rel_lo && key <= rel_hi;
      x[r] = ok ? st[r] * p.scale_log2 : kNegInf;
      tmax = fmaxf(tmax, x[r]);
    }
    tmax = fmaxf(tmax, shfl_xor(tmax, 32));
    // Lazy rescale: the reference max m_run moves only when the tile's max
    // exceeds it by more than 8 (log2 units), so the probabilities stay below
    // 2^8 and O (in AGPRs: a read, a multiply and a write per element) is
    // rescaled only then -- after the first tile of a window almost never.
    // exp2(x - m) / sum exp2(x - m) is the same softmax for any reference m.
    const float m_new = tmax > m_run + 8.f ? tmax : m_run;
    const float m_use = m_new == kNegInf ? 0.f : m_new;   // nothing seen yet: every term is 0
    const float alpha = fast_exp2(m_run - m_use);          // 0 on the first keys (O and z are 0)
    float psum = 0.f;
    bf16x8 pb[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float e = fast_exp2(x[r] - m_use);
      psum += e;
      pb[r >> 3][r & 7] = to_bf16(e);
    }
    z_run = z_run * alpha + psum;
    // O is still 0 while m_run is -inf: no rescale needed then
    const bool rescale = alpha != 1.f && m_run != kNegInf;
    m_run = m_new;
    if (__builtin_amdgcn_ballot_w64(rescale) != 0) {
#pragma unroll
      for (int n = 0; n < 8; ++n) oacc[n] *= alpha;
    }
    // O^T += V^T P^T: A = V^T (dims 32n + l32, keys in the register order of P);
    // step j = (ks, n) = (j / 8, j % 8)
    auto vfrag = [&](int j) {
      const int krow = 16 * (j >> 3) + 4 * (G >> 1) + (s16 >> 2);
      const int col = 32 * (j & 7) + 16 * (G & 1) + 4 * (s16 & 3);
      const bf16* v0 = (const bf16*)(vb + krow * SW_VP) + col;
      const bf16* v1 = (const bf16*)(vb + (krow + 8) * SW_VP) + col;
      return cat8(lds_tr16(v0), lds_tr16(v1));
    };
    bf16x8 vf[16];
#pragma unroll
    for (int j = 0; j < SW_AHEAD; ++j) vf[j] = vfrag(j);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      oacc[j & 7] = mfma32(vf[j], pb[j >> 3], oacc[j & 7]);
      if (j + SW_AHEAD < 16) vf[j + SW_AHEAD] = vfrag(j + SW_AHEAD);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Tile kt sits in buffer (kt - kt0) % 2; after the barrier that makes it
  // visible, every wave is also done with tile kt - 1, so the DMA of tile kt+1
  // into that buffer is issued right away and lands while tile kt computes.
  // The buffers are picked at run time: one copy of the loop body, so that the
  // accumulators keep their registers from one tile to the next.
  for (int kt = kt0; kt <= kt1; ++kt) {
    const bool odd = (kt - kt0) & 1;
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's DMA of tile kt
    __syncthreads();
    if (kt < kt1) dma(kt + 1, odd ? lds_k0 : lds_k1, odd ? lds_v0 : lds_v1);
    step(kt, odd ? lds_k1 : lds_k0, odd ? lds_v1 : lds_v0);
  }

  // ---- outputs: lane l holds O[row l32][32n + 8(r/4) + 4hb + r%4].  The
  // normalised bf16 rows go to the wave's staging buffer (pitch 33 chunks: the
  // 8-byte writes of 16 rows hit distinct banks), then out as whole rows.
  const float z = z_run + shfl_xor(z_run, 32);
  const float inv = z > 0.f ? 1.f / z : 0.f;
  if (hb == 0 && row_ok && p.lse) p.lse[q_row] = z > 0.f ? (m_run + fast_log2(z)) * kLn2 : kNegInf;
  __syncthreads();   // every wave is done with the last tile
#pragma unroll
  for (int n = 0; n < 8; ++n)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      bf16x4 w;
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = to_bf16(oacc[n][4 * a + j] * inv);
      *(bf16x4*)(wbuf + l32 * SW_KP + 64 * n + 16 * a + 8 * hb) = w;
    }
  // instruction j: rows 2j (lanes 0..31) and 2j + 1 (lanes 32..63), 16 B a lane
  const __amdgpu_buffer_rsrc_t ro = rows_rsrc(p.o);
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int row = 2 * j + hb;
    const u32x4 v = *(const u32x4*)(wbuf + row * SW_KP + 16 * l32);
    __builtin_amdgcn_raw_buffer_store_b128(v, ro, row * 512 + 16 * l32, 0, 0);
  }
}

}  // namespace

hipError_t launch_rope(RopeParams p, double rope_base, hipStream_t stream) {
  // frequency of pair m in revolutions per position: base^(-2m/R) / (2 pi)
  for (int m = 0; m < p.rope_dims / 2; ++m)
    p.rev[m] = std::pow(rope_base, -2.0 * m / p.rope_dims) / (2.0 * 3.14159265358979323846);
  const bool inplace = p.x == p.y;
  if (inplace && p.rope_dims == 0) return hipSuccess;
  const int64_t chunks = p.n_rows * (inplace ? p.rope_dims / 8 : 32);
  const dim3 grid((unsigned)((chunks + 255) / 256));
  if (inplace)
    hipLaunchKernelGGL(rope_kernel<true>, grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(rope_kernel<false>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_swa(const SwaParams& p, hipStream_t stream) {
  const int tpb = SW_WAVES * 32 / p.H;
  const unsigned nblk = (unsigned)((int64_t)p.B * ((p.n_q + tpb - 1) / tpb));
  switch (p.H) {
    case 1: hipLaunchKernelGGL(swa_kernel<1>, dim3(nblk), dim3(SW_THREADS), 0, stream, p); break;
    case 2: hipLaunchKernelGGL(swa_kernel<2>, dim3(nblk), dim3(SW_THREADS), 0, stream, p); break;
    case 4: hipLaunchKernelGGL(swa_kernel<4>, dim3(nblk), dim3(SW_THREADS), 0, stream, p); break;
    case 8: hipLaunchKernelGGL(swa_kernel<8>, dim3(nblk), dim3(SW_THREADS), 0, stream, p); break;
    default: hipLaunchKernelGGL(swa_kernel<16>, dim3(nblk), dim3(SW_THREADS), 0, stream, p); break;
  }
  return hipGetLastError();
}

}  // namespace hs2

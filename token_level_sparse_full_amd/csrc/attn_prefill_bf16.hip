// Scored full attention, many-query path, bf16 caches.
//
// Same definition and the same two sweeps as attn_prefill.hip (HySparse2
// pages, agihunt.info summary: the full layer's exact attention probabilities
// score the tokens for the sparse layers; per head P_hj = exp(l_hj - lse_h),
// score_j = sum_h P_hj), laid out for MI355X as two kernels over the same
// 256-row workgroups (64 query rows per wave = 64/H tokens x H heads):
//
//  * prefill_lse: S^T = K Q^T per 32-key tile (a lane owns a row, online
//    max/sum in registers) -> lse of every row (log2 units, workspace).  It
//    holds no O accumulator, so two workgroups share a CU and the two waves of
//    a SIMD hide each other's LDS and MFMA latency; K tiles are triple-buffered.
//  * prefill_pv: S = Q K^T (a lane owns a key: float32 P from the lse, in-lane
//    head sums for the scores), P -> LDS [key][row] -> transposed reads ->
//    O += P V.  The 64 x 256 float32 O accumulator of a wave fills the AGPR
//    file (one wave per SIMD); with 16 heads all 64 query rows of the wave
//    stay in VGPRs (with fewer heads rows 32..63 are parked in LDS), and
//    operands are read three MFMA steps ahead of their use.
//
// Both stream K (and V) in 32-key tiles through LDS with global_load_lds_dwordx4
// (no register staging), one barrier per tile.  Every buffer is its own LDS
// object and the loops are unrolled over the buffers, so that the compiler
// sees that reads of one buffer do not depend on the DMA into another.  Every
// K or V fragment read from LDS feeds two 32-row MFMA tiles, which halves the
// LDS bytes per MFMA flop against 32-row waves.
#include <algorithm>
#include <type_traits>

#include "hs2_device.hpp"
#include "hs2_internal.hpp"

namespace hs2 {
namespace {

constexpr int PB_WAVES = 4;
constexpr int PB_THREADS = PB_WAVES * kWave;
constexpr int PB_KT = 32;                       // keys per tile
constexpr int PB_RW = 64;                       // rows per wave
// LDS rows are padded rather than swizzled, so that every operand read of a
// lane is one base register plus an immediate offset:
//   K rows: 33 chunks of 16 B (528 B): 16 consecutive rows read at the same
//           chunk hit 16 distinct 4-bank groups;
//   V rows: 34 chunks (544 B): the 4 rows x 32 B of one transposed read hit
//           32 distinct banks.
constexpr int PB_KC = 33, PB_VC = 34;           // chunks per padded K / V row
constexpr int PB_KTILE = 17 * 1024;             // 32 x 33 chunks (16.5 KB) rounded to 17 DMA instructions
constexpr int PB_VTILE = 17 * 1024;             // 32 x 34 chunks = 17 DMA instructions
constexpr int PB_PP = 144;                      // P buffer pitch (bytes per key)
constexpr int PB_AHEAD = 3;                     // operand prefetch distance (MFMA steps)

// 32x32x16 bf16 MFMAs whose accumulator is pinned to VGPRs.  The P/V kernel
// keeps its 64 x 256 float32 O accumulator in the 256 AGPRs; a builtin MFMA for
// S would also be given AGPRs and the compiler would shuffle O tiles in and out
// of VGPRs every tile.  Written as inline asm, the S accumulators stay in VGPRs.
// The compiler inserts no hazard wait states around inline asm, so each block
// carries its own (gfx950, 8-pass XDL):
//  * before each MFMA, 3 wait states cover a VALU write of an A/B operand;
//  * the last block of a chain ends with 20 wait states, more than an XDL
//    result needs before a VALU, LDS or memory instruction may read it.
// Back-to-back MFMAs on the same accumulator need none.  LDS loads feeding the
// operands are covered by the compiler's s_waitcnt insertion (it sees asm uses).
// The other direction matters too: an XDL op keeps reading its A and B
// registers after it issues, so nothing may overwrite them right away (a VALU
// write one instruction after the MFMA has been seen to corrupt S).  For the
// compiler an asm operand is dead once the asm has issued, so each MFMA takes
// the operands of the MFMA before it as unused inputs (ka, kb): they stay
// allocated until this one issues, at least one full MFMA (32 cycles) later.
// tests/test_asm_hazards.py checks the compiled code for both directions.
__device__ __forceinline__ void mfma32v_first(f32x16& acc, bf16x8 a, bf16x8 b) {
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma32v_first(f32x16& acc, bf16x8 a, bf16x8 b, bf16x8 ka) {
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b), "v"(ka));
}
__device__ __forceinline__ void mfma32v(f32x16& acc, bf16x8 a, bf16x8 b, bf16x8 ka, bf16x8 kb) {
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b), "v"(ka), "v"(kb));
}
// last step of two chains sharing the B operand, then the read-after-write
// wait (which also covers the operand reads of both)
__device__ __forceinline__ void mfma32v_last2(f32x16& acc0, f32x16& acc1, bf16x8 a0, bf16x8 a1, bf16x8 b, bf16x8 ka,
                                              bf16x8 kb) {
  asm volatile(
      "s_nop 2\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %2, %4, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %1, %3, %4, %1\n\t"
      "s_nop 7\n\ts_nop 7\n\ts_nop 3"
      : "+v"(acc0), "+v"(acc1)
      : "v"(a0), "v"(a1), "v"(b), "v"(ka), "v"(kb));
}

// PHASE 1: prefill_lse, PHASE 2: prefill_pv.  SC: the K and V rows come with
// per-row float32 scales (an e4m3 cache widened to bf16 codes): a logit is
// S * (scale * k_scale[key]) and P is multiplied by v_scale[key] before it is
// rounded to bf16 for the PV product, the arithmetic of the e4m3 path of
// attn_prefill.hip; each tile's scales ride along with its K or V DMA.
template <int H, int PHASE, bool SC>
__global__ __launch_bounds__(PB_THREADS, PHASE == 1 ? 2 : 1) void prefill_bf16_kernel(const AttnParams p, float* lse2) {
  constexpr int TPW = PB_RW / H;       // tokens per wave
  constexpr int TPB = PB_WAVES * TPW;  // tokens per workgroup

  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int hb = l >> 5, l32 = l & 31;
  const int G = l >> 4, s16 = l & 15;

  const int nblk_tok = (p.n_q + TPB - 1) / TPB;
  const int b = blockIdx.x / nblk_tok;
  const int tb = nblk_tok - 1 - (blockIdx.x % nblk_tok);  // latest (heaviest) token blocks first
  const int tok_blk0 = tb * TPB;
  const int tok_w0 = tok_blk0 + wave * TPW;
  const int n_valid_blk = min(TPB, p.n_q - tok_blk0);
  const int64_t pos_first = p.q_pos0 + tok_blk0;
  const int64_t n_keys = pos_first + n_valid_blk;
  const int ntiles = (int)((n_keys + PB_KT - 1) / PB_KT);
  const char* kg = (const char*)p.k + (int64_t)b * p.T * 512;
  const char* vg = (const char*)p.v + (int64_t)b * p.T * 512;
  const int64_t q_row0 = ((int64_t)b * p.n_q + tok_w0) * H;   // first query row of this wave

  auto tok_of_row = [&](int row) { return tok_w0 + row / H; };
  auto pos_of_row = [&](int row) -> int64_t {
    const int t = tok_of_row(row);
    return p.q_pos0 + (t < p.n_q ? t : p.n_q - 1);
  };
  // query row 32*mt + l32 of this wave, K-step s: dims 16s + 8hb .. +7
  auto qload = [&](int mt, int s) -> u32x4 {
    const bool ok = tok_of_row(32 * mt + l32) < p.n_q;
    const bf16* qp = (const bf16*)p.q + (q_row0 + 32 * mt + l32) * kHeadDim + 8 * hb;
    return ok ? *(const u32x4*)(qp + 16 * s) : u32x4{0u, 0u, 0u, 0u};
  };

  // ---- LDS DMA of one 32-key tile into its padded image: the image is cut into
  // 17 wave-instructions of 64 x 16 B (lane l of instruction i fills chunk
  // 64 i + l); instruction i is issued by wave i % 4.  Pad chunks and the slack
  // after the last row load a valid row and are never read.  The per-lane
  // source offsets inside a tile are loop invariant.  The loads go through a
  // buffer resource that ends at the tile's last valid key, so rows past it
  // read as zeros (and are masked later).  Buffer loads to LDS rather than
  // global_load_lds: after the latter the compiler can no longer count LDS
  // reads in order and waits for all of them at every use.
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  uint32_t koff[5], voff[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int c = 64 * (wv + 4 * i) + l;
    const int kr = c / PB_KC, kc = c - kr * PB_KC;
    const int vr = c / PB_VC, vc = c - vr * PB_VC;
    koff[i] = (uint32_t)(min(kr, PB_KT - 1) * 512 + (kc < 32 ? kc : 0) * 16);
    voff[i] = (uint32_t)(min(vr, PB_KT - 1) * 512 + (vc < 32 ? vc : 0) * 16);
  }
  // buffer resource over the valid rows of tile kt (none past the last key):
  // loads past them return 0
  auto tile_rsrc = [&](const char* g, int kt) __attribute__((always_inline)) {
    const int64_t rows = max((int64_t)0, min((int64_t)PB_KT, n_keys - (int64_t)kt * PB_KT));
    return __builtin_amdgcn_make_buffer_rsrc((void*)(g + (int64_t)kt * (PB_KT * 512)), 0, (int)(rows * 512), 0x00020000);
  };
  // DMA instruction i (0..4) of this wave for one tile image
  auto dma_one = [&](const __amdgpu_buffer_rsrc_t& rs, char* buf, const uint32_t (&off)[5], int i) __attribute__((always_inline)) {
    const int ins = wv + 4 * i;
    if (i < 4 || (i == 4 && wv == 0))   // 17 instructions: wave 0 issues the last one
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (void HS2_LDS*)((char HS2_LDS*)buf + ins * 1024), 16, off[i], 0, 0, 0);
  };
  auto dma = [&](const char* g, int kt, char* buf, const uint32_t (&off)[5]) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(g, kt);
#pragma unroll
    for (int i = 0; i < 5; ++i) dma_one(rs, buf, off, i);
  };
  auto wait_dma = [] { __builtin_amdgcn_s_waitcnt(0x0F70); };  // vmcnt(0)
  // the 32 row scales of tile kt (zeros past the last key) -> sc[0..31], by
  // one DMA instruction of 4 bytes per lane (lanes 32..63 land in sc[32..63],
  // never read)
  auto dma_scales = [&](const float* src, int kt, float* sc) __attribute__((always_inline)) {
    const int64_t rows = max((int64_t)0, min((int64_t)PB_KT, n_keys - (int64_t)kt * PB_KT));
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(src + (int64_t)b * p.T + (int64_t)kt * PB_KT), 0, (int)(rows * 4), 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (void HS2_LDS*)sc, 4, (uint32_t)(4 * l), 0, 0, 0);
  };
  // K fragment for K-step s: key l32 of the tile, dims 16s + 8hb .. +7
  const int kofs = l32 * (PB_KC * 16) + 16 * hb;
  auto kfrag = [&](const char* buf, int s) -> bf16x8 { return as_bf16x8(*(const u32x4*)(buf + kofs + 32 * s)); };

  struct Pair {
    f32x16 v[2];
  };

  if constexpr (PHASE == 1) {
    // =============================== prefill_lse ===============================
    __shared__ __attribute__((aligned(1024))) char lds_k0[PB_KTILE], lds_k1[PB_KTILE], lds_k2[PB_KTILE];
    __shared__ __attribute__((aligned(16))) float lds_ks[SC ? 3 : 1][64];   // K row scales of each buffer
    bf16x8 qf[2][16];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int s = 0; s < 16; ++s) qf[mt][s] = as_bf16x8(qload(mt, s));
    float m_run[2] = {kNegInf, kNegInf}, z_run[2] = {0.f, 0.f};
    const int my_pos[2] = {(int)pos_of_row(l32), (int)pos_of_row(32 + l32)};
    // Online max / sum of one tile (lane: rows l32 and 32 + l32, keys kt*32 +
    // 8(r/4) + 4hb + r%4); cf[r] is the logit factor of key r: the softmax
    // scale in log2 units, times the key's row scale in the scaled form.
    // Tiles left of the diagonal need no causal mask: that path is the bulk of
    // the work, so it is kept free of selects.
    //
    // Left of the diagonal the running maximum is a lazy reference: a tile's
    // exponentials are taken against it as it stands, and it is raised (with
    // the rescale of the sum) only when a tile's sum of 16 terms per row
    // block exceeds 2^64, i.e. when some logit lies more than 60 (log2 units)
    // above it.  The terms stay below 2^64 and the sum below 2^81, far inside
    // float32, and terms far below the reference underflow as they would
    // against the true maximum; the sum carries the same relative rounding
    // either way.  This drops the tile maximum (16 max per row block) from
    // the common case.  The test is wave-uniform: if any lane fails it, the
    // whole wave redoes the tile against the true maximum.
    auto lse_update = [&](Pair& st, int kt, bool masked, const float (&cf)[16]) __attribute__((always_inline)) {
      const int kbase = kt * PB_KT;
      if (!masked) {
        float accl[2];
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          float a = 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) a += fast_exp2(st.v[n][r] * cf[r] - m_run[n]);
          accl[n] = a;
        }
        // !(a <= 2^64) also catches a first tile (m_run = -inf: a = +inf)
        if (!__any(!(accl[0] <= 0x1p64f) || !(accl[1] <= 0x1p64f))) {
          z_run[0] += accl[0];
          z_run[1] += accl[1];
          return;
        }
      }
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        float tmax = kNegInf;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = st.v[n][r] * cf[r];
          if (masked) x = (kbase + 8 * (r >> 2) + 4 * hb + (r & 3) <= my_pos[n]) ? x : kNegInf;
          st.v[n][r] = x;
          tmax = fmaxf(tmax, x);
        }
        const float m_new = fmaxf(m_run[n], tmax);
        const float m_use = m_new == kNegInf ? 0.f : m_new;  // all masked so far: every term is 0
        float acc = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc += fast_exp2(st.v[n][r] - m_use);
        z_run[n] = z_run[n] * fast_exp2(m_run[n] - m_use) + acc;   // exp2(-inf) = 0 on the first tile
        m_run[n] = m_new;
      }
    };
    // Tile kt sits in kc; K(kt+2) goes to kd, which held K(kt-1) (past the last
    // tile the buffer resource is empty and the DMA writes zeros, so that every
    // tile issues the same instructions).  K(kt+1) may still be in flight at
    // the wait: each wave keeps its last batch of DMA instructions (5 for wave
    // 0, 4 for the others, 5 for wave 1 in the scaled form, which also carries
    // the tile's 32 K row scales) outstanding.  The batch is spread over the
    // first ten MFMA steps (one instruction every second step): issued that
    // early it has landed by the wait two tiles later.  In the scaled form the
    // factors of tile kt are read from its scale buffer ksc after the MFMAs
    // (the DMA that reuses that buffer is issued in the next step).
    auto step1 = [&](int kt, const char* kc, char* kd, const float* ksc, float* ksd) __attribute__((always_inline)) {
      if (wv == 0 || (SC && wv == 1)) __builtin_amdgcn_s_waitcnt(0x0F75);   // vmcnt(5)
      else __builtin_amdgcn_s_waitcnt(0x0F74);                              // vmcnt(4)
      __syncthreads();
      const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kg, kt + 2);
      Pair st;
      bf16x8 kf[16];
#pragma unroll
      for (int s = 0; s < PB_AHEAD; ++s) kf[s] = kfrag(kc, s);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        st.v[0] = mfma32(kf[s], qf[0][s], s == 0 ? f32x16{} : st.v[0]);
        if (s + PB_AHEAD < 16) kf[s + PB_AHEAD] = kfrag(kc, s + PB_AHEAD);
        st.v[1] = mfma32(kf[s], qf[1][s], s == 0 ? f32x16{} : st.v[1]);
        if (s % 2 == 0 && s < 10) dma_one(rk, kd, koff, s / 2);
        if constexpr (SC) {
          if (s == 10 && wv == 1) dma_scales(p.k_scale, kt + 2, ksd);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_sched_barrier(0);
      float cf[16];
      if constexpr (SC) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 c4 = *(const f32x4*)(ksc + 8 * q + 4 * hb);
#pragma unroll
          for (int e = 0; e < 4; ++e) cf[4 * q + e] = c4[e] * p.scale_log2;
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) cf[r] = p.scale_log2;
      }
      lse_update(st, kt, (int64_t)kt * PB_KT + PB_KT - 1 > pos_first, cf);
    };
    {
      float* const ks0 = lds_ks[0];
      float* const ks1 = lds_ks[SC ? 1 : 0];
      float* const ks2 = lds_ks[SC ? 2 : 0];
      // issue order per wave: K(0), scales(0), K(1), scales(1), so that the
      // first wait (all but the last batch) covers tile 0 and its scales
      dma(kg, 0, lds_k0, koff);
      if (SC && wv == 1) dma_scales(p.k_scale, 0, ks0);
      dma(kg, 1, lds_k1, koff);
      if (SC && wv == 1) dma_scales(p.k_scale, 1, ks1);
      int kt = 0;
      for (; kt + 2 < ntiles; kt += 3) {
        step1(kt, lds_k0, lds_k2, ks0, ks2);
        step1(kt + 1, lds_k1, lds_k0, ks1, ks0);
        step1(kt + 2, lds_k2, lds_k1, ks2, ks1);
      }
      if (kt < ntiles) step1(kt, lds_k0, lds_k2, ks0, ks2);
      if (kt + 1 < ntiles) step1(kt + 1, lds_k1, lds_k0, ks1, ks0);
      wait_dma();   // the zero-filling DMA past the last tile
    }
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const float mo = shfl_xor(m_run[n], 32), zo = shfl_xor(z_run[n], 32);
      const float m = fmaxf(m_run[n], mo);
      const float z = (m_run[n] == kNegInf ? 0.f : z_run[n] * fast_exp2(m_run[n] - m)) +
                      (mo == kNegInf ? 0.f : zo * fast_exp2(mo - m));
      if (hb == 0 && tok_of_row(32 * n + l32) < p.n_q) {
        const float l2 = m + fast_log2(z);
        lse2[q_row0 + 32 * n + l32] = l2;
        if (p.lse) p.lse[q_row0 + 32 * n + l32] = l2 * kLn2;
      }
    }
  } else {
    // =============================== prefill_pv ===============================
    __shared__ __attribute__((aligned(1024))) char lds_k0[PB_KTILE], lds_k1[PB_KTILE];
    __shared__ __attribute__((aligned(1024))) char lds_v0[PB_VTILE], lds_v1[PB_VTILE];
    __shared__ __attribute__((aligned(16))) char lds_p[PB_WAVES * PB_KT * PB_PP];
    __shared__ __attribute__((aligned(16))) float lds_lse[PB_WAVES * PB_RW];
    __shared__ __attribute__((aligned(16))) float lds_ksc[SC ? 2 : 1][64], lds_vsc[SC ? 2 : 1][64];   // by tile parity
    char* const pbuf = lds_p + wave * PB_KT * PB_PP;
    float* const lse_lds = lds_lse + wave * PB_RW;
    // With H = 16 all 64 query rows of the wave stay in registers (128 VGPRs),
    // so the S block reads only K from LDS.  The smaller H run out of
    // registers that way: their rows 32..63 go to LDS as [s][lane] (16 KB per
    // wave), so that each fragment read is one conflict-free ds_read_b128.
    constexpr bool QREG = H == 16;
    __shared__ __attribute__((aligned(1024))) char lds_q[QREG ? 16 : PB_WAVES * 16 * 1024];
    char* const qlds = lds_q + (QREG ? 0 : wave * (16 * 1024) + l * 16);
    bf16x8 qf[16], qf1[QREG ? 16 : 1];
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      qf[s] = as_bf16x8(qload(0, s));
      if constexpr (QREG)
        qf1[s] = as_bf16x8(qload(1, s));
      else
        *(u32x4*)(qlds + s * 1024) = qload(1, s);
    }
    auto q1frag = [&](int s) -> bf16x8 { return as_bf16x8(*(const u32x4*)(qlds + s * 1024)); };
    // lse of the wave's rows (log2 units); rows past the last token read row 0's
    if (l < PB_RW) {
      const int64_t r = tok_of_row(l) < p.n_q ? q_row0 + l : q_row0;
      lse_lds[l] = lse2[r];
    }
    __syncthreads();

    // =============================== sweep 2: P, scores, O ===============================
    f32x16 oacc[2][8];
  #pragma unroll
    for (int mt = 0; mt < 2; ++mt)
  #pragma unroll
      for (int n = 0; n < 8; ++n) oacc[mt][n] = f32x16{};
    float* srow_base = p.scores + (int64_t)b * p.n_q * p.ld_scores;
    // S = Q K^T (lane = key l32, regs = rows), operands PB_AHEAD steps ahead;
    // hook(s) runs inside step s (the next tile's DMA, the scores)
    auto s_rows_keys = [&](const char* kb, auto hook) __attribute__((always_inline)) {
      Pair sa;
      bf16x8 kf[16], q1[QREG ? 1 : 16];
  #pragma unroll
      for (int s = 0; s < PB_AHEAD; ++s) {
        kf[s] = kfrag(kb, s);
        if constexpr (!QREG) q1[s] = q1frag(s);
      }
      // rows 32..63, K-step s: from registers, or prefetched from LDS
      auto q1op = [&](int s) -> bf16x8 {
        if constexpr (QREG) return qf1[s]; else return q1[s];
      };
      __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
      for (int s = 0; s < 16; ++s) {
        // the A chain keeps the previous step's B-chain operands alive, the B
        // chain those of the A chain before it
        if (s == 15) {
          mfma32v_last2(sa.v[0], sa.v[1], qf[s], q1op(s), kf[s], q1op(s - 1), kf[s - 1]);
        } else {
          if (s == 0) mfma32v_first(sa.v[0], qf[s], kf[s]); else mfma32v(sa.v[0], qf[s], kf[s], q1op(s - 1), kf[s - 1]);
          if (s + PB_AHEAD < 16) kf[s + PB_AHEAD] = kfrag(kb, s + PB_AHEAD);
          if (s == 0) mfma32v_first(sa.v[1], q1op(s), kf[s], qf[s]); else mfma32v(sa.v[1], q1op(s), kf[s], qf[s], kf[s]);
          if constexpr (!QREG) {
            if (s + PB_AHEAD < 16) q1[s + PB_AHEAD] = q1frag(s + PB_AHEAD);
          }
        }
        hook(s);
        __builtin_amdgcn_sched_barrier(0);
      }
      return sa;
    };

    // scores of tile kt to global memory (token sums of 32/H tokens per 32-row tile)
    auto store_scores = [&](const Pair& sa, int kt, const float (&sc)[2][2]) __attribute__((always_inline)) {
      const int64_t key = (int64_t)kt * PB_KT + l32;
  #pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        auto put = [&](int row_in_tile0, float val) {
          const int tok = tok_of_row(32 * mt + row_in_tile0);
          if (tok < p.n_q && key <= p.q_pos0 + tok) srow_base[(int64_t)tok * p.ld_scores + key] = val;
        };
        if constexpr (H == 16) {
          put(16 * hb, sc[mt][0]);
        } else if constexpr (H == 8) {
          put(8 * hb, sc[mt][0]);
          put(16 + 8 * hb, sc[mt][1]);
        } else if constexpr (H == 4) {
  #pragma unroll
          for (int q = 0; q < 4; ++q)
            put(8 * q + 4 * hb, sa.v[mt][4 * q] + sa.v[mt][4 * q + 1] + sa.v[mt][4 * q + 2] + sa.v[mt][4 * q + 3]);
        } else if constexpr (H == 2) {
  #pragma unroll
          for (int q = 0; q < 4; ++q)
  #pragma unroll
            for (int jj = 0; jj < 2; ++jj)
              put(8 * q + 4 * hb + 2 * jj, sa.v[mt][4 * q + 2 * jj] + sa.v[mt][4 * q + 2 * jj + 1]);
        } else {
  #pragma unroll
          for (int r = 0; r < 16; ++r) put(8 * (r >> 2) + 4 * hb + (r & 3), sa.v[mt][r]);
        }
      }
    };
    // A operands of O += P V (P rows x keys, transposed reads of the [key][row]
    // buffer), all four read at once so that the buffer is free for the next P.
    auto read_pa = [&](const char* pb, bf16x8 (&a)[2][2]) __attribute__((always_inline)) {
  #pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int krow = 16 * ks + 8 * (G >> 1) + (s16 >> 2);
        const int off = 16 * (G & 1) + 4 * (s16 & 3);
  #pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const bf16* pa = (const bf16*)(pb + krow * PB_PP) + 32 * mt + off;
          a[ks][mt] = cat8(lds_tr16(pa), lds_tr16(pa + 4 * (PB_PP / 2)));
        }
      }
    };
    // V fragment of PV step j = (ks, n) = (j / 8, j % 8): keys 16 ks + ..., dims 32 n + ...
    auto read_b = [&](const char* vb, int j) __attribute__((always_inline)) {
      const int ks = j >> 3, n = j & 7;
      const int krow = 16 * ks + 8 * (G >> 1) + (s16 >> 2);
      const int off = 16 * (G & 1) + 4 * (s16 & 3);
      const bf16* vrow = (const bf16*)(vb + krow * (PB_VC * 16)) + off;
      return cat8(lds_tr16(vrow + 32 * n), lds_tr16(vrow + 4 * (PB_VC * 8) + 32 * n));
    };
    // O += P V for the last tile alone (V fragments PB_AHEAD steps ahead)
    auto pv_only = [&](const bf16x8 (&a)[2][2], const char* vb) __attribute__((always_inline)) {
      bf16x8 bv[16];
  #pragma unroll
      for (int j = 0; j < PB_AHEAD; ++j) bv[j] = read_b(vb, j);
      __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int ks = j >> 3, n = j & 7;
        oacc[0][n] = mfma32(a[ks][0], bv[j], oacc[0][n]);
        if (j + PB_AHEAD < 16) bv[j + PB_AHEAD] = read_b(vb, j + PB_AHEAD);
        oacc[1][n] = mfma32(a[ks][1], bv[j], oacc[1][n]);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // The probabilities of tile kt woven into the 16 steps of O += P(kt-1) V(kt-1)
    // (two MFMAs per step, with_pv) or alone (first tile).  Step s handles the
    // logits r = 4q + 2(s%2) + {0,1} of row block mt = s/8, q = (s/2)%4 (lane:
    // key kbase + l32, rows 32mt + 8q + 4hb + j): exp2 against the row lse, then
    // at the end of a q group P (bf16) -> LDS [key][row], at the end of a row
    // block the head sums of the scores.  The order is fixed per step, so that
    // at most PB_AHEAD V fragments and two lse vectors are in flight.
    auto pv_probs = [&](const bf16x8 (&a)[2][2], const char* vb, Pair& sa, int kt, char* pb, float (&sc)[2][2],
                        auto masked, auto with_pv, auto hook) __attribute__((always_inline)) {
      constexpr bool need_mask = decltype(masked)::value;
      constexpr bool do_pv = decltype(with_pv)::value;
      const int64_t key = (int64_t)kt * PB_KT + l32;
      auto lse4 = [&](int g) { return *(const f32x4*)(lse_lds + 32 * (g >> 2) + 8 * (g & 3) + 4 * hb); };
      // logit factor of this lane's key, and its V scale (SC)
      float cl = p.scale_log2, vsl = 1.f;
      if constexpr (SC) {
        cl = p.scale_log2 * lds_ksc[kt & 1][l32];
        vsl = lds_vsc[kt & 1][l32];
      }
      bf16x8 bv[16];
      if constexpr (do_pv) {
  #pragma unroll
        for (int j = 0; j < PB_AHEAD; ++j) bv[j] = read_b(vb, j);
      }
      f32x4 lcur = lse4(0), lnext = lse4(1);
      __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
      for (int st = 0; st < 16; ++st) {
        if constexpr (do_pv) {
          const int ks = st >> 3, n = st & 7;
          oacc[0][n] = mfma32(a[ks][0], bv[st], oacc[0][n]);
          if (st + PB_AHEAD < 16) bv[st + PB_AHEAD] = read_b(vb, st + PB_AHEAD);
          oacc[1][n] = mfma32(a[ks][1], bv[st], oacc[1][n]);
        }
        const int g = st >> 1, mt = st >> 3, q = g & 3;
  #pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int j = 2 * (st & 1) + jj, r = 4 * q + j;
          const float e = fast_exp2(sa.v[mt][r] * cl - lcur[j]);
          if constexpr (need_mask)
            sa.v[mt][r] = key <= pos_of_row(32 * mt + 8 * q + 4 * hb + j) ? e : 0.f;
          else
            sa.v[mt][r] = e;
        }
        if (st & 1) {
          bf16x4 v4;
          if constexpr (SC) {
            v4[0] = to_bf16(sa.v[mt][4 * q] * vsl);
            v4[1] = to_bf16(sa.v[mt][4 * q + 1] * vsl);
            v4[2] = to_bf16(sa.v[mt][4 * q + 2] * vsl);
            v4[3] = to_bf16(sa.v[mt][4 * q + 3] * vsl);
          } else {
            v4[0] = to_bf16(sa.v[mt][4 * q]);
            v4[1] = to_bf16(sa.v[mt][4 * q + 1]);
            v4[2] = to_bf16(sa.v[mt][4 * q + 2]);
            v4[3] = to_bf16(sa.v[mt][4 * q + 3]);
          }
          *(bf16x4*)(pb + l32 * PB_PP + (32 * mt + 8 * q + 4 * hb) * 2) = v4;
          lcur = lnext;
          if (g + 2 < 8) lnext = lse4(g + 2);
        }
        if ((st & 7) == 7) {
          if constexpr (H == 16) {
            float t0 = 0.f, t1 = 0.f;
  #pragma unroll
            for (int r = 0; r < 8; ++r) {
              t0 += sa.v[mt][r];
              t1 += sa.v[mt][8 + r];
            }
            sc[mt][0] = halfwave_pair_sum(t0, t1);
          } else if constexpr (H == 8) {
            float t[4];
  #pragma unroll
            for (int qq = 0; qq < 4; ++qq)
              t[qq] = sa.v[mt][4 * qq] + sa.v[mt][4 * qq + 1] + sa.v[mt][4 * qq + 2] + sa.v[mt][4 * qq + 3];
            sc[mt][0] = halfwave_pair_sum(t[0], t[1]);
            sc[mt][1] = halfwave_pair_sum(t[2], t[3]);
          }
        }
        hook(st);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // Sweep 2, software-pipelined over tiles: iteration t computes S(t), then
    // the probabilities of tile t on the VALU while the MFMAs compute
    // O += P(t-1) V(t-1).  Iteration t waits for K(t) and V(t-1) (issued in
    // iteration t-1), then fetches K(t+1) and V(t): V is one tile behind K, so
    // two buffers of each suffice.  P(t-1) is read into registers before P(t)
    // overwrites the wave's P buffer.  With H >= 8 the scores of a tile are
    // written one tile late, right after the DMA issue, so that the stores have
    // long completed when the next wait on the vector-memory counter comes.
    float sc_prev[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
    auto finish_scores = [&](const Pair& sa, int kt, const float (&sc)[2][2]) __attribute__((always_inline)) {
      if constexpr (H >= 8) {
  #pragma unroll
        for (int mt = 0; mt < 2; ++mt) sc_prev[mt][0] = sc[mt][0], sc_prev[mt][1] = sc[mt][1];
      } else {
        store_scores(sa, kt, sc);
      }
    };
    // Start of tile kt: K(kt) and V(kt-1) have landed.  P(kt-1) is already in
    // registers: the P buffer is the wave's own, so it is read at the end of
    // the previous tile, before the barrier, and its read latency stays off
    // the path from the barrier to the first MFMA.
    auto sync_tile = [&]() __attribute__((always_inline)) {
      wait_dma();
      __syncthreads();
    };
    bf16x8 pa[2][2];
    // The DMA of K(kt+1) (zeros past the last tile) and of V(kt) both go in
    // the S steps, one instruction of each every third step: a CU moves about
    // 46 bytes per clock into LDS, and a burst would stall the issuing wave.
    // Issued this early, V(kt) has landed by the next wait (issuing it in the
    // PV steps left about 0.4 k cycles of that wait per tile).
    auto iter = [&](int kt, const char* kc, char* kn, const char* vp, char* vn, auto masked) __attribute__((always_inline)) {
      sync_tile();
      const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kg, kt + 1), rv = tile_rsrc(vg, kt);
      Pair sa = s_rows_keys(kc, [&](int st) __attribute__((always_inline)) {
        if (st % 3 == 0 && st < 15) dma_one(rk, kn, koff, st / 3);
        if (st % 3 == 1 && st < 14) dma_one(rv, vn, voff, st / 3);
        if constexpr (SC) {
          // the scales of tile kt + 1, used by its probabilities in the next
          // iteration (after that iteration's wait and barrier)
          if (st == 14 && wv == 1) dma_scales(p.k_scale, kt + 1, lds_ksc[SC ? ((kt + 1) & 1) : 0]);
          if (st == 14 && wv == 2) dma_scales(p.v_scale, kt + 1, lds_vsc[SC ? ((kt + 1) & 1) : 0]);
        }
        if constexpr (H >= 8) {
          if (st == 14) store_scores(Pair{}, kt - 1, sc_prev);
        }
      });
      float sc[2][2];
      pv_probs(pa, vp, sa, kt, pbuf, sc, masked, std::true_type{}, [](int) {});
      finish_scores(sa, kt, sc);
      read_pa(pbuf, pa);   // P(kt), for the next tile
    };
    // first tile is never preceded by a PV block
    const int t_mask = (int)((pos_first + 1) / PB_KT);   // tiles >= t_mask need the causal mask
    dma(kg, 0, lds_k0, koff);
    if constexpr (SC) {
      if (wv == 1) dma_scales(p.k_scale, 0, lds_ksc[0]);
      if (wv == 2) dma_scales(p.v_scale, 0, lds_vsc[0]);
    }
    {
      bf16x8 none[2][2] = {};
      sync_tile();
      if (ntiles > 1) dma(kg, 1, lds_k1, koff);
      dma(vg, 0, lds_v0, voff);
      if constexpr (SC) {
        if (wv == 1) dma_scales(p.k_scale, 1, lds_ksc[SC ? 1 : 0]);
        if (wv == 2) dma_scales(p.v_scale, 1, lds_vsc[SC ? 1 : 0]);
      }
      Pair sa = s_rows_keys(lds_k0, [](int) {});
      float sc[2][2];
      if (t_mask == 0)
        pv_probs(none, lds_v0, sa, 0, pbuf, sc, std::true_type{}, std::false_type{}, [](int) {});
      else
        pv_probs(none, lds_v0, sa, 0, pbuf, sc, std::false_type{}, std::false_type{}, [](int) {});
      finish_scores(sa, 0, sc);
      read_pa(pbuf, pa);
    }
    {
      int kt = 1;
      for (; kt + 1 < t_mask; kt += 2) {
        iter(kt, lds_k1, lds_k0, lds_v0, lds_v1, std::false_type{});
        iter(kt + 1, lds_k0, lds_k1, lds_v1, lds_v0, std::false_type{});
      }
      if (kt < t_mask) {
        iter(kt, lds_k1, lds_k0, lds_v0, lds_v1, std::false_type{});
        ++kt;
      }
      // The few tiles on the diagonal pick their buffers at run time: one copy
      // of the body, and no register pressure from two unrolled copies.
      for (; kt < ntiles; ++kt) {
        const bool odd = kt & 1;
        iter(kt, odd ? lds_k1 : lds_k0, odd ? lds_k0 : lds_k1, odd ? lds_v0 : lds_v1, odd ? lds_v1 : lds_v0,
             std::true_type{});
      }
    }
    // last PV block
    wait_dma();
    __syncthreads();
    if constexpr (H >= 8) store_scores(Pair{}, ntiles - 1, sc_prev);
    pv_only(pa, ((ntiles - 1) & 1) ? lds_v1 : lds_v0);

    // ---- outputs: lane holds O[32mt + 8(r/4) + 4hb + r%4][32n + l32]
  #pragma unroll
    for (int mt = 0; mt < 2; ++mt)
  #pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * mt + 8 * (r >> 2) + 4 * hb + (r & 3);
        if (tok_of_row(row) >= p.n_q) continue;
        bf16* orow = (bf16*)p.o + (q_row0 + row) * kHeadDim;
  #pragma unroll
        for (int n = 0; n < 8; ++n) orow[32 * n + l32] = to_bf16(oacc[mt][n][r]);
      }
  }
}

}  // namespace

// workspace: the lse of every row (log2 units); with an e4m3 cache also the
// cache widened to bf16 codes, K then V, [B][T][256] each
size_t prefill_bf16_workspace_bytes(int B, int n_q, int H, int64_t T, bool e4m3) {
  const size_t lse = ((size_t)B * n_q * H * 4 + 255) & ~(size_t)255;
  return e4m3 ? lse + 2 * (size_t)B * T * 512 : lse;
}

// e4m3 codes -> bf16 codes (exact: every e4m3 value is a bf16 value), 16 per thread
__global__ __launch_bounds__(256) void widen_e4m3_kernel(const uint32_t* src, bf16* dst, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256) {
    const u32x4 c = __builtin_nontemporal_load((const u32x4*)src + i);
    *(bf16x8*)(dst + 16 * i) = e4m3x8_to_bf16(c[0], c[1]);
    *(bf16x8*)(dst + 16 * i + 8) = e4m3x8_to_bf16(c[2], c[3]);
  }
}

template <int H, bool SC>
hipError_t launch_prefill_bf16_h(const AttnParams& p, float* lse2, hipStream_t stream) {
  const int tpb = PB_WAVES * PB_RW / H;
  const unsigned nblk = (unsigned)(p.B * ((p.n_q + tpb - 1) / tpb));
  hipLaunchKernelGGL((prefill_bf16_kernel<H, 1, SC>), dim3(nblk), dim3(PB_THREADS), 0, stream, p, lse2);
  hipLaunchKernelGGL((prefill_bf16_kernel<H, 2, SC>), dim3(nblk), dim3(PB_THREADS), 0, stream, p, lse2);
  return hipGetLastError();
}

template <bool SC>
hipError_t launch_prefill_bf16_sc(const AttnParams& p, float* lse2, hipStream_t stream) {
  switch (p.H) {
    case 1: return launch_prefill_bf16_h<1, SC>(p, lse2, stream);
    case 2: return launch_prefill_bf16_h<2, SC>(p, lse2, stream);
    case 4: return launch_prefill_bf16_h<4, SC>(p, lse2, stream);
    case 8: return launch_prefill_bf16_h<8, SC>(p, lse2, stream);
    default: return launch_prefill_bf16_h<16, SC>(p, lse2, stream);
  }
}

hipError_t launch_prefill_bf16(const AttnParams& p, void* ws, hipStream_t stream, bool e4m3) {
  float* lse2 = (float*)ws;
  if (!e4m3) return launch_prefill_bf16_sc<false>(p, lse2, stream);
  // widen the e4m3 cache into the workspace, then run the bf16 passes on it
  const size_t lse_bytes = prefill_bf16_workspace_bytes(p.B, p.n_q, p.H, p.T, false);
  bf16* kw = (bf16*)((char*)ws + lse_bytes);
  bf16* vw = kw + (size_t)p.B * p.T * 256;
  const int64_t n16 = (int64_t)p.B * p.T * 16;
  const unsigned grid = (unsigned)std::min<int64_t>((n16 + 255) / 256, 8192);
  hipLaunchKernelGGL(widen_e4m3_kernel, dim3(grid), dim3(256), 0, stream, (const uint32_t*)p.k, kw, n16);
  hipLaunchKernelGGL(widen_e4m3_kernel, dim3(grid), dim3(256), 0, stream, (const uint32_t*)p.v, vw, n16);
  AttnParams q = p;
  q.k = kw;
  q.v = vw;
  return launch_prefill_bf16_sc<true>(q, lse2, stream);
}

}  // namespace hs2

// 16-row attention tiles shared by the decode (split over keys) and sparse
// reuse kernels.  Up to 16 query rows (the heads of one MQA token, or a few
// tokens times their heads) form the N axis of 16x16 MFMA tiles:
//   S^T (keys x rows) = K Q^T,    O^T (dims x rows) += V^T P^T.
// A lane l of a wave owns row c16 = l % 16 and, inside a 16-key tile, the keys
// 4*(l/16) + r, r = 0..3, of S^T; the same lane owns row c16 of O^T.
//
// Head-dim mapping of the contraction (K and Q fragments must agree):
//   bf16 cache, K-step s, lane group g:  d = 32 s + 8 g + i
//   e4m3 cache, K-step s:                d = 64 (s/2) + 16 g + 8 (s%2) + i
//   f32 cache, chunk cs, element j:      d = 16 cs + 4 g + j  (16x16x4 MFMA)
// V rows of a step sit row-major in LDS (bf16, or f32 for the f32 cache) and
// feed the dims x keys operand through ds_read_b64_tr_b16 (bf16) or plain
// 4-byte reads (f32).
#pragma once

#include "hs2_device.hpp"

namespace hs2 {

template <int KV>
struct TileCfg {
  static constexpr int STEP = 32;     // keys per step (two 16-key tiles)
  static constexpr int PITCH = 272;   // LDS row pitch in elements (544 B: rows shift by 8 banks)
};
template <>
struct TileCfg<KV_F32> {
  static constexpr int STEP = 16;
  static constexpr int PITCH = 260;   // floats
};
constexpr int kTileStageBytes = 32 * 272 * 2;  // also holds 16 x 260 floats
static_assert(16 * 260 * 4 <= kTileStageBytes, "f32 stage");

struct QFrag {
  bf16x8 b[8];
  f32x4 f[16];
};

// Query fragment of row `qrow` (pointer to its 256 elements) for this lane.
template <int KV>
__device__ __forceinline__ void load_qfrag(const void* qrow, bool ok, int g, QFrag& qf) {
  if constexpr (KV == KV_F32) {
    const float* qp = (const float*)qrow;
#pragma unroll
    for (int cs = 0; cs < 16; ++cs) qf.f[cs] = ok ? *(const f32x4*)(qp + 16 * cs + 4 * g) : f32x4{0.f, 0.f, 0.f, 0.f};
  } else {
    const bf16* qp = (const bf16*)qrow;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int d0 = (KV == KV_BF16) ? 32 * s + 8 * g : 64 * (s >> 1) + 16 * g + 8 * (s & 1);
      qf.b[s] = ok ? as_bf16x8(*(const u32x4*)(qp + d0)) : as_bf16x8(u32x4{0u, 0u, 0u, 0u});
    }
  }
}

// One 16x16 tile of S^T for the 16 keys of this lane's tile row (`krow` is
// the K row of key c16 of the tile, or nullptr for an absent key).
template <int KV>
__device__ __forceinline__ f32x4 s_tile(const void* krow, int g, const QFrag& qf) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const bool ok = krow != nullptr;
  if constexpr (KV == KV_F32) {
    const float* kp = (const float*)krow;
    f32x4 kf[16];
#pragma unroll
    for (int cs = 0; cs < 16; ++cs) kf[cs] = ok ? *(const f32x4*)(kp + 16 * cs + 4 * g) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cs = 0; cs < 16; ++cs)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc = mfma16_f32(kf[cs][j], qf.f[cs][j], acc);
  } else if constexpr (KV == KV_BF16) {
    const bf16* kp = (const bf16*)krow;
    bf16x8 kf[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) kf[s] = ok ? as_bf16x8(*(const u32x4*)(kp + 32 * s + 8 * g)) : as_bf16x8(u32x4{0u, 0u, 0u, 0u});
#pragma unroll
    for (int s = 0; s < 8; ++s) acc = mfma16(kf[s], qf.b[s], acc);
  } else {
    const uint8_t* kp = (const uint8_t*)krow;
    u32x4 raw[4];
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) raw[s2] = ok ? *(const u32x4*)(kp + 64 * s2 + 16 * g) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      acc = mfma16(e4m3x8_to_bf16(raw[s2][0], raw[s2][1]), qf.b[2 * s2], acc);
      acc = mfma16(e4m3x8_to_bf16(raw[s2][2], raw[s2][3]), qf.b[2 * s2 + 1], acc);
    }
  }
  return acc;
}

// Stage the V rows of one step into LDS.  rowptr(slot) returns the V row of
// step slot `slot` (0..STEP-1) or nullptr for an absent key.
template <int KV, typename RowPtr>
__device__ __forceinline__ void stage_v(char* stage, int l, RowPtr rowptr) {
  constexpr int PITCH = TileCfg<KV>::PITCH;
  if constexpr (KV == KV_F32) {
    float* stg = (float*)stage;
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const float* vp = (const float*)rowptr(it);
      const f32x4 val = vp ? *(const f32x4*)(vp + 4 * l) : f32x4{0.f, 0.f, 0.f, 0.f};
      *(f32x4*)(stg + it * PITCH + 4 * l) = val;
    }
  } else if constexpr (KV == KV_BF16) {
    bf16* stg = (bf16*)stage;
    u32x4 val[16];
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const bf16* vp = (const bf16*)rowptr(2 * it + (l >> 5));
      val[it] = vp ? *(const u32x4*)(vp + 8 * (l & 31)) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int it = 0; it < 16; ++it) *(u32x4*)(stg + (2 * it + (l >> 5)) * PITCH + 8 * (l & 31)) = val[it];
  } else {
    bf16* stg = (bf16*)stage;
    u32x4 val[8];
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const uint8_t* vp = (const uint8_t*)rowptr(4 * it + (l >> 4));
      val[it] = vp ? *(const u32x4*)(vp + 16 * (l & 15)) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      bf16* dst = stg + (4 * it + (l >> 4)) * PITCH + 16 * (l & 15);
      *(bf16x8*)dst = e4m3x8_to_bf16(val[it][0], val[it][1]);
      *(bf16x8*)(dst + 8) = e4m3x8_to_bf16(val[it][2], val[it][3]);
    }
  }
}

// O^T += V^T P^T for one step.  pr[mt][r] is the (already V-scaled)
// probability of key slot 16mt + 4g + r for this lane's row.
template <int KV>
__device__ __forceinline__ void pv_step(const char* stage, const float (&pr)[TileCfg<KV>::STEP / 16][4], int g, int c16,
                                        f32x4 (&oacc)[16]) {
  constexpr int PITCH = TileCfg<KV>::PITCH;
  if constexpr (KV == KV_F32) {
    const float* stg = (const float*)stage;
#pragma unroll
    for (int t = 0; t < 16; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) oacc[t] = mfma16_f32(stg[(4 * g + j) * PITCH + 16 * t + c16], pr[0][j], oacc[t]);
  } else {
    bf16x8 pb;
#pragma unroll
    for (int i = 0; i < 8; ++i) pb[i] = to_bf16(pr[i >> 2][i & 3]);  // slot 8g+i <-> key 16(i/4) + 4g + i%4
    const bf16* stg = (const bf16*)stage;
    const bf16* r_lo = stg + (4 * g + (c16 >> 2)) * PITCH + 4 * (c16 & 3);
    const bf16* r_hi = r_lo + 16 * PITCH;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const bf16x8 a = cat8(lds_tr16(r_lo + 16 * t), lds_tr16(r_hi + 16 * t));
      oacc[t] = mfma16(a, pb, oacc[t]);
    }
  }
}

__device__ __forceinline__ void wave_lds_order() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

}  // namespace hs2

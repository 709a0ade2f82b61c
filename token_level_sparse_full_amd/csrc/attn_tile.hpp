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

// Register counts of one tile's K fragment and of one step's V rows per lane
// (loaded first, consumed later, so that the loads of one step can be in
// flight while the previous step computes).
template <int KV>
struct FragRegs {
  static constexpr int K = (KV == KV_E4M3) ? 4 : (KV == KV_BF16 ? 8 : 16);  // u32x4 per 16-key tile
  static constexpr int V = (KV == KV_E4M3) ? 8 : 16;                        // u32x4 per step
};

// This lane's K fragment of one 16-key tile; `krow` is the K row of key c16
// of the tile and must be readable (an absent key is given some valid row,
// and its logit masked later, so the loads need no branch).
template <int KV>
__device__ __forceinline__ void load_k_tile(const void* krow, int g, u32x4* kr) {
  if constexpr (KV == KV_F32) {
    const float* kp = (const float*)krow;
#pragma unroll
    for (int cs = 0; cs < 16; ++cs) kr[cs] = *(const u32x4*)(kp + 16 * cs + 4 * g);
  } else if constexpr (KV == KV_BF16) {
    const bf16* kp = (const bf16*)krow;
#pragma unroll
    for (int s = 0; s < 8; ++s) kr[s] = *(const u32x4*)(kp + 32 * s + 8 * g);
  } else {
    const uint8_t* kp = (const uint8_t*)krow;
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) kr[s2] = *(const u32x4*)(kp + 64 * s2 + 16 * g);
  }
}

// One 16x16 tile of S^T from a loaded K fragment.
template <int KV>
__device__ __forceinline__ f32x4 s_from_k(const u32x4* kr, const QFrag& qf) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if constexpr (KV == KV_F32) {
#pragma unroll
    for (int cs = 0; cs < 16; ++cs) {
      const f32x4 kf = __builtin_bit_cast(f32x4, kr[cs]);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc = mfma16_f32(kf[j], qf.f[cs][j], acc);
    }
  } else if constexpr (KV == KV_BF16) {
#pragma unroll
    for (int s = 0; s < 8; ++s) acc = mfma16(as_bf16x8(kr[s]), qf.b[s], acc);
  } else {
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      acc = mfma16(e4m3x8_to_bf16(kr[s2][0], kr[s2][1]), qf.b[2 * s2], acc);
      acc = mfma16(e4m3x8_to_bf16(kr[s2][2], kr[s2][3]), qf.b[2 * s2 + 1], acc);
    }
  }
  return acc;
}

// One 16x16 tile of S^T for the 16 keys of this lane's tile row (`krow` is
// nullptr for an absent key: zeros).
template <int KV>
__device__ __forceinline__ f32x4 s_tile(const void* krow, int g, const QFrag& qf) {
  u32x4 kr[FragRegs<KV>::K];
#pragma unroll
  for (int i = 0; i < FragRegs<KV>::K; ++i) kr[i] = u32x4{0u, 0u, 0u, 0u};
  if (krow != nullptr) load_k_tile<KV>(krow, g, kr);
  return s_from_k<KV>(kr, qf);
}

// This lane's share of the V rows of one step.  rowptr(slot) returns the V
// row of step slot `slot` (0..STEP-1); with NULLABLE it may return nullptr
// for an absent key (zeros), else it must return a readable row.
template <int KV, bool NULLABLE, typename RowPtr>
__device__ __forceinline__ void load_v_rows(int l, RowPtr rowptr, u32x4* vr) {
  const u32x4 z = {0u, 0u, 0u, 0u};
  auto ld = [&](const char* vp, int off) -> u32x4 {
    if constexpr (NULLABLE) return vp ? *(const u32x4*)(vp + off) : z;
    return *(const u32x4*)(vp + off);
  };
  if constexpr (KV == KV_F32) {
#pragma unroll
    for (int it = 0; it < 16; ++it) vr[it] = ld((const char*)rowptr(it), 16 * l);
  } else if constexpr (KV == KV_BF16) {
#pragma unroll
    for (int it = 0; it < 16; ++it) vr[it] = ld((const char*)rowptr(2 * it + (l >> 5)), 16 * (l & 31));
  } else {
#pragma unroll
    for (int it = 0; it < 8; ++it) vr[it] = ld((const char*)rowptr(4 * it + (l >> 4)), 16 * (l & 15));
  }
}

// Write the loaded V rows into the LDS stage (row-major, bf16 or f32).
template <int KV>
__device__ __forceinline__ void store_v_rows(char* stage, int l, const u32x4* vr) {
  constexpr int PITCH = TileCfg<KV>::PITCH;
  if constexpr (KV == KV_F32) {
    float* stg = (float*)stage;
#pragma unroll
    for (int it = 0; it < 16; ++it) *(u32x4*)(stg + it * PITCH + 4 * l) = vr[it];
  } else if constexpr (KV == KV_BF16) {
    bf16* stg = (bf16*)stage;
#pragma unroll
    for (int it = 0; it < 16; ++it) *(u32x4*)(stg + (2 * it + (l >> 5)) * PITCH + 8 * (l & 31)) = vr[it];
  } else {
    bf16* stg = (bf16*)stage;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      bf16* dst = stg + (4 * it + (l >> 4)) * PITCH + 16 * (l & 15);
      *(bf16x8*)dst = e4m3x8_to_bf16(vr[it][0], vr[it][1]);
      *(bf16x8*)(dst + 8) = e4m3x8_to_bf16(vr[it][2], vr[it][3]);
    }
  }
}

// K rows of a step as whole rows (loaded with load_v_rows, so that each load
// instruction covers whole cache lines) -> LDS -> MFMA fragments.  Fragment
// reads of 16 rows at one offset hit distinct banks at these pitches (bf16
// 528 B, e4m3 codes 272 B: rows shift by 4 banks).  The bf16 image (16.5 KB)
// fits the V stage, which the same wave fills after reading the fragments.
template <int KV>
struct KStage {
  static constexpr int PITCH_B = KV == KV_BF16 ? 528 : 272;
};
static_assert(32 * 528 <= kTileStageBytes, "K stage");
template <int KV>
__device__ __forceinline__ void store_k_rows(char* stage, int l, const u32x4* kr) {
  constexpr int PB = KStage<KV>::PITCH_B;
  if constexpr (KV == KV_BF16) {
#pragma unroll
    for (int it = 0; it < 16; ++it) *(u32x4*)(stage + (2 * it + (l >> 5)) * PB + 16 * (l & 31)) = kr[it];
  } else {
#pragma unroll
    for (int it = 0; it < 8; ++it) *(u32x4*)(stage + (4 * it + (l >> 4)) * PB + 16 * (l & 15)) = kr[it];
  }
}
// This lane's K fragment of 16-key tile mt of the staged rows (the layout of
// load_k_tile).
template <int KV>
__device__ __forceinline__ void read_k_tile(const char* stage, int mt, int c16, int g, u32x4* kr) {
  const char* row = stage + (16 * mt + c16) * KStage<KV>::PITCH_B;
  if constexpr (KV == KV_BF16) {
#pragma unroll
    for (int s = 0; s < 8; ++s) kr[s] = *(const u32x4*)(row + (32 * s + 8 * g) * 2);
  } else {
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) kr[s2] = *(const u32x4*)(row + 64 * s2 + 16 * g);
  }
}

// Stage the V rows of one step into LDS.
template <int KV, typename RowPtr>
__device__ __forceinline__ void stage_v(char* stage, int l, RowPtr rowptr) {
  u32x4 vr[FragRegs<KV>::V];
  load_v_rows<KV, true>(l, rowptr, vr);
  store_v_rows<KV>(stage, l, vr);
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

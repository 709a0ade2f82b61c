// Scored full attention, many-query path (prefill chunks).
//
// HySparse2 pages, agihunt.info summary: the full-attention layer of the
// cross-decoder is exact MQA attention with NoPE and also acts as the selector,
// scoring tokens with its exact attention probabilities for the sparse layers
// that follow.  Per query at position p and head h:
//   l_j = scale <q_h, k_j> (j <= p),  P_hj = exp(l_j - lse_h),
//   o_h = sum_j P_hj v_j,  score_j = sum_h P_hj.
//
// The scores need the final per-head normaliser before any probability is
// formed, so the kernel runs two sweeps over the causal keys of its queries:
//   sweep 1: S^T = K Q^T  (keys x rows): a lane owns one (token, head) row and
//            keeps an online max / sum for it in registers -> lse per row;
//   sweep 2: S = Q K^T   (rows x keys): a lane owns one key and sees 16 rows,
//            so P = exp2(S*c - lse2) in float32 and the head sum of the score is
//            an in-lane add plus one half-wave swap; P (bf16) goes to LDS as
//            [key][row] and comes back through ds_read_b64_tr_b16 as the A
//            operand of O += P V, with V read transposed the same way.
// The rows of a wave are 32/H tokens x H heads (MQA: every head of every
// token reads the same K/V tile).  Workgroup: 4 waves = 128 rows; key tiles of
// 64 (32 for float32) are staged in LDS with XOR-swizzled 16-byte chunks and
// prefetched into registers one tile ahead.  Only float32 caches use this
// kernel: bf16 caches, and e4m3 caches widened to bf16 codes, run the
// LDS-DMA pipeline of attn_prefill_bf16.hip.
#include "hs2_device.hpp"
#include "hs2_internal.hpp"

namespace hs2 {
namespace {

constexpr int PF_WAVES = 4;
constexpr int PF_THREADS = PF_WAVES * kWave;

template <int KV>
struct PfCfg {
  static constexpr bool F32 = (KV == KV_F32);
  static constexpr int KT = F32 ? 32 : 64;          // keys per tile
  static constexpr int ROWB = F32 ? 1024 : 512;     // bytes per K/V row (LDS and HBM)
  static constexpr int GROWB = ROWB;
  static constexpr int GCPR = GROWB / 16;           // 16-byte chunks per row
  static constexpr int LOADS = KT * GROWB / 16 / PF_THREADS;  // 16-byte loads per thread per tile
  static constexpr int P_PITCH = F32 ? 144 : 72;    // bytes per key row of the P buffer
  static constexpr int P_BYTES = KT * P_PITCH;
};

constexpr int kPfSmem = 2 * 32768 + PF_WAVES * 64 * 72 + PF_WAVES * 32 * 4;
static_assert(PF_WAVES * 32 * 144 <= PF_WAVES * 64 * 72, "f32 P buffer fits");

__device__ __forceinline__ int k_swz(int row, int ch) { return ch ^ (row & 15); }
__device__ __forceinline__ int v_swz(int row, int ch) { return ch ^ (2 * (row & 3)); }

template <int KV, int H>
__global__ __launch_bounds__(PF_THREADS, 1) void prefill_kernel(const AttnParams p) {
  using C = PfCfg<KV>;
  constexpr int KT = C::KT;
  constexpr int TPW = 32 / H;          // tokens per wave
  constexpr int TPB = PF_WAVES * TPW;  // tokens per workgroup
  constexpr int NJ = KT / 32;          // 32-key sub-tiles per tile
  __shared__ __attribute__((aligned(16))) char smem[kPfSmem];
  char* k_lds = smem;
  char* v_lds = smem + 32768;
  char* p_lds_all = smem + 65536;
  float* lse_lds_all = (float*)(p_lds_all + PF_WAVES * 64 * 72);

  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int hb = l >> 5, l32 = l & 31;
  const int G = l >> 4, s16 = l & 15;

  // heaviest (latest) token blocks first for a short causal tail
  const int nblk_tok = (p.n_q + TPB - 1) / TPB;
  const int b = blockIdx.x / nblk_tok;
  const int tb = nblk_tok - 1 - (blockIdx.x % nblk_tok);
  const int tok_blk0 = tb * TPB;
  const int tok_w0 = tok_blk0 + wave * TPW;
  const int n_valid_blk = min(TPB, p.n_q - tok_blk0);
  const int64_t pos_first = p.q_pos0 + tok_blk0;
  const int64_t n_keys = pos_first + n_valid_blk;  // keys 0 .. last position of the block
  const int ntiles = (int)((n_keys + KT - 1) / KT);
  const int64_t kv_row0 = (int64_t)b * p.T;
  char* p_lds = p_lds_all + wave * 64 * 72;
  float* lse_lds = lse_lds_all + wave * 32;

  auto tok_of_row = [&](int row) { return tok_w0 + row / H; };
  auto pos_of_row = [&](int row) {
    const int t = tok_of_row(row);
    return p.q_pos0 + (t < p.n_q ? t : p.n_q - 1);
  };

  // ---- queries of this wave's 32 rows (row = token_local * H + head)
  const int64_t q_row0 = ((int64_t)b * p.n_q + tok_w0) * H;  // first row of the wave
  const bool my_row_ok = tok_of_row(l32) < p.n_q;
  bf16x8 qf[16];
  f32x4 qf32[32];
  if constexpr (C::F32) {
    const float* qp = (const float*)p.q + (q_row0 + l32) * kHeadDim + 4 * hb;
#pragma unroll
    for (int cs = 0; cs < 32; ++cs) qf32[cs] = my_row_ok ? *(const f32x4*)(qp + 8 * cs) : f32x4{0.f, 0.f, 0.f, 0.f};
  } else {
    const bf16* qp = (const bf16*)p.q + (q_row0 + l32) * kHeadDim + 8 * hb;
#pragma unroll
    for (int s = 0; s < 16; ++s)
      qf[s] = my_row_ok ? as_bf16x8(*(const u32x4*)(qp + 16 * s)) : as_bf16x8(u32x4{0u, 0u, 0u, 0u});
  }

  // ---- tile staging: global -> registers -> LDS (swizzled)
  const char* kg = (const char*)p.k + kv_row0 * C::GROWB;
  const char* vg = (const char*)p.v + kv_row0 * C::GROWB;
  auto load_tile = [&](const char* base, int kt, u32x4* r) {
#pragma unroll
    for (int it = 0; it < C::LOADS; ++it) {
      const int c = it * PF_THREADS + tid;
      const int row = c / C::GCPR, ch = c % C::GCPR;
      const int64_t key = (int64_t)kt * KT + row;
      r[it] = key < n_keys ? *(const u32x4*)(base + key * C::GROWB + ch * 16) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto put_chunk = [&](char* lds, int row, int ch, u32x4 x, bool vlayout) {
    auto swz = [&](int c) { return vlayout ? (C::F32 ? c : v_swz(row, c)) : k_swz(row, c); };
    *(u32x4*)(lds + row * C::ROWB + swz(ch) * 16) = x;
  };
  auto store_k = [&](const u32x4* r) {
#pragma unroll
    for (int it = 0; it < C::LOADS; ++it) {
      const int c = it * PF_THREADS + tid;
      put_chunk(k_lds, c / C::GCPR, c % C::GCPR, r[it], false);
    }
  };
  auto store_v = [&](const u32x4* r) {
#pragma unroll
    for (int it = 0; it < C::LOADS; ++it) {
      const int c = it * PF_THREADS + tid;
      put_chunk(v_lds, c / C::GCPR, c % C::GCPR, r[it], true);
    }
  };
  // K fragment of key row `key` (tile-local) for K-step s (bf16) / chunk-step cs (f32)
  auto k_frag = [&](int key, int ch) -> u32x4 {
    return *(const u32x4*)(k_lds + key * C::ROWB + k_swz(key, ch) * 16);
  };

  // =============================== sweep 1: lse per row ===============================
  float m_run = kNegInf, z_run = 0.f;
  const int64_t my_pos = pos_of_row(l32);
  u32x4 stg[2 * C::LOADS];
  load_tile(kg, 0, stg);
  for (int kt = 0; kt < ntiles; ++kt) {
    __syncthreads();
    store_k(stg);
    __syncthreads();
    if (kt + 1 < ntiles) load_tile(kg, kt + 1, stg);
    f32x16 sacc[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      sacc[j] = f32x16{};
      const int key = 32 * j + l32;
      if constexpr (C::F32) {
#pragma unroll
        for (int cs = 0; cs < 32; ++cs) {
          const f32x4 kv4 = __builtin_bit_cast(f32x4, k_frag(key, 2 * cs + hb));
#pragma unroll
          for (int e = 0; e < 4; ++e) sacc[j] = mfma32_f32(kv4[e], qf32[cs][e], sacc[j]);
        }
      } else {
#pragma unroll
        for (int s = 0; s < 16; ++s) sacc[j] = mfma32(as_bf16x8(k_frag(key, 2 * s + hb)), qf[s], sacc[j]);
      }
    }
    // lane: row l32, keys 32j + 8(r/4) + 4hb + r%4
    const int64_t kbase = (int64_t)kt * KT;
    const bool need_mask = kbase + KT - 1 > pos_first;
    float tmax = kNegInf;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = sacc[j][r] * p.scale_log2;
        if (need_mask) {
          const int64_t key = kbase + 32 * j + 8 * (r >> 2) + 4 * hb + (r & 3);
          x = key <= my_pos ? x : kNegInf;
        }
        sacc[j][r] = x;
        tmax = fmaxf(tmax, x);
      }
    const float m_new = fmaxf(m_run, tmax);
    if (m_new != kNegInf) {
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc += fast_exp2(sacc[j][r] - m_new);  // exp2(-inf) = 0
      z_run = z_run * fast_exp2(m_run - m_new) + acc;
      m_run = m_new;
    }
  }
  {
    // merge the two lane halves that share a row
    const float mo = shfl_xor(m_run, 32), zo = shfl_xor(z_run, 32);
    const float m = fmaxf(m_run, mo);
    const float z = (m_run == kNegInf ? 0.f : z_run * fast_exp2(m_run - m)) + (mo == kNegInf ? 0.f : zo * fast_exp2(mo - m));
    if (hb == 0) lse_lds[l32] = m + fast_log2(z);
  }
  __syncthreads();
  // rows seen by this lane in sweep 2: 8(r/4) + 4hb + r%4
  float lse2[16];
  int64_t rpos[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = 8 * (r >> 2) + 4 * hb + (r & 3);
    lse2[r] = lse_lds[row];
    rpos[r] = pos_of_row(row);
  }

  // =============================== sweep 2: P, scores, O ===============================
  f32x16 oacc[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) oacc[n] = f32x16{};
  float* srow_base = p.scores + ((int64_t)b * p.n_q) * p.ld_scores;

  load_tile(kg, 0, stg);
  load_tile(vg, 0, stg + C::LOADS);
  for (int kt = 0; kt < ntiles; ++kt) {
    __syncthreads();
    store_k(stg);
    store_v(stg + C::LOADS);
    __syncthreads();
    if (kt + 1 < ntiles) {
      load_tile(kg, kt + 1, stg);
      load_tile(vg, kt + 1, stg + C::LOADS);
    }
    const int64_t kbase = (int64_t)kt * KT;
    const bool need_mask = kbase + KT - 1 > pos_first;
    f32x16 sacc[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      sacc[j] = f32x16{};
      const int key = 32 * j + l32;
      if constexpr (C::F32) {
#pragma unroll
        for (int cs = 0; cs < 32; ++cs) {
          const f32x4 kv4 = __builtin_bit_cast(f32x4, k_frag(key, 2 * cs + hb));
#pragma unroll
          for (int e = 0; e < 4; ++e) sacc[j] = mfma32_f32(qf32[cs][e], kv4[e], sacc[j]);
        }
      } else {
#pragma unroll
        for (int s = 0; s < 16; ++s) sacc[j] = mfma32(qf[s], as_bf16x8(k_frag(key, 2 * s + hb)), sacc[j]);
      }
    }
    // probabilities (lane: key 32j + l32, rows 8(r/4) + 4hb + r%4)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int64_t key = kbase + 32 * j + l32;
      const float c = p.scale_log2;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = fast_exp2(sacc[j][r] * c - lse2[r]);
        sacc[j][r] = (!need_mask || key <= rpos[r]) ? e : 0.f;
      }
    }
    // ---- scores: sum over the H rows of each token
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int64_t key = kbase + 32 * j + l32;
      auto put = [&](int tok_local, float val) {
        const int tok = tok_w0 + tok_local;
        if (tok < p.n_q && key <= p.q_pos0 + tok) srow_base[(int64_t)tok * p.ld_scores + key] = val;
      };
      if constexpr (H == 16) {
        float t0 = 0.f, t1 = 0.f;
#pragma unroll
        for (int r = 0; r < 8; ++r) { t0 += sacc[j][r]; t1 += sacc[j][8 + r]; }
        put(hb, halfwave_pair_sum(t0, t1));
      } else if constexpr (H == 8) {
        float t[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) t[q] = sacc[j][4 * q] + sacc[j][4 * q + 1] + sacc[j][4 * q + 2] + sacc[j][4 * q + 3];
        put(hb, halfwave_pair_sum(t[0], t[1]));
        put(2 + hb, halfwave_pair_sum(t[2], t[3]));
      } else if constexpr (H == 4) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          put(2 * q + hb, sacc[j][4 * q] + sacc[j][4 * q + 1] + sacc[j][4 * q + 2] + sacc[j][4 * q + 3]);
      } else if constexpr (H == 2) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) put(4 * q + 2 * hb + jj, sacc[j][4 * q + 2 * jj] + sacc[j][4 * q + 2 * jj + 1]);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) put(8 * (r >> 2) + 4 * hb + (r & 3), sacc[j][r]);
      }
    }
    // ---- P -> LDS as [key][row]
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int key = 32 * j + l32;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row0 = 8 * q + 4 * hb;
        if constexpr (C::F32) {
          const f32x4 v4 = {sacc[j][4 * q], sacc[j][4 * q + 1], sacc[j][4 * q + 2], sacc[j][4 * q + 3]};
          *(f32x4*)(p_lds + key * C::P_PITCH + row0 * 4) = v4;
        } else {
          bf16x4 v4;
          v4[0] = to_bf16(sacc[j][4 * q]);
          v4[1] = to_bf16(sacc[j][4 * q + 1]);
          v4[2] = to_bf16(sacc[j][4 * q + 2]);
          v4[3] = to_bf16(sacc[j][4 * q + 3]);
          *(bf16x4*)(p_lds + key * C::P_PITCH + row0 * 2) = v4;
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    // ---- O += P V
    if constexpr (C::F32) {
#pragma unroll
      for (int kp = 0; kp < KT / 2; ++kp) {
        const int key = 2 * kp + hb;
        const float a = *(const float*)(p_lds + key * C::P_PITCH + l32 * 4);
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          const float bv = *(const float*)(v_lds + key * C::ROWB + (32 * n + l32) * 4);
          oacc[n] = mfma32_f32(a, bv, oacc[n]);
        }
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < KT / 16; ++ks) {
        const int kb = 16 * ks + 8 * (G >> 1) + (s16 >> 2);
        const int colp = 16 * (G & 1) + 4 * (s16 & 3);   // row offset inside the P row / column offset in V
        const bf16* pa = (const bf16*)(p_lds + kb * C::P_PITCH) + colp;
        const bf16x8 a = cat8(lds_tr16(pa), lds_tr16(pa + 4 * (C::P_PITCH / 2)));
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          const int col = 32 * n + colp;            // bf16 column in the V row
          const int ch = col >> 3, half = (col >> 2) & 1;
          const char* v0 = v_lds + kb * C::ROWB + v_swz(kb, ch) * 16 + half * 8;
          const char* v1 = v_lds + (kb + 4) * C::ROWB + v_swz(kb + 4, ch) * 16 + half * 8;
          const bf16x8 bv = cat8(lds_tr16((const bf16*)v0), lds_tr16((const bf16*)v1));
          oacc[n] = mfma32(a, bv, oacc[n]);
        }
      }
    }
  }

  // ---- outputs: O (lane: column 32n + l32, rows 8(r/4) + 4hb + r%4) and lse
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = 8 * (r >> 2) + 4 * hb + (r & 3);
    if (tok_of_row(row) >= p.n_q) continue;
    const int64_t orow = (q_row0 + row) * kHeadDim;
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      if constexpr (C::F32)
        ((float*)p.o)[orow + 32 * n + l32] = oacc[n][r];
      else
        ((bf16*)p.o)[orow + 32 * n + l32] = to_bf16(oacc[n][r]);
    }
  }
  if (p.lse && hb == 0 && my_row_ok) p.lse[q_row0 + l32] = lse_lds[l32] * kLn2;
}

template <int KV>
hipError_t launch_prefill_kv(const AttnParams& p, hipStream_t stream) {
  const int tpb = PF_WAVES * 32 / p.H;
  const unsigned nblk = (unsigned)(p.B * ((p.n_q + tpb - 1) / tpb));
  switch (p.H) {
    case 1: hipLaunchKernelGGL((prefill_kernel<KV, 1>), dim3(nblk), dim3(PF_THREADS), 0, stream, p); break;
    case 2: hipLaunchKernelGGL((prefill_kernel<KV, 2>), dim3(nblk), dim3(PF_THREADS), 0, stream, p); break;
    case 4: hipLaunchKernelGGL((prefill_kernel<KV, 4>), dim3(nblk), dim3(PF_THREADS), 0, stream, p); break;
    case 8: hipLaunchKernelGGL((prefill_kernel<KV, 8>), dim3(nblk), dim3(PF_THREADS), 0, stream, p); break;
    default: hipLaunchKernelGGL((prefill_kernel<KV, 16>), dim3(nblk), dim3(PF_THREADS), 0, stream, p); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const AttnParams& p, void* ws, hipStream_t stream, bool e4m3);  // attn_prefill_bf16.hip

hipError_t launch_prefill(const AttnParams& p, int kv_kind, void* ws, hipStream_t stream) {
  if (p.B * p.n_q == 0) return hipSuccess;
  switch (kv_kind) {
    case KV_F32: return launch_prefill_kv<KV_F32>(p, stream);
    // e4m3: widened to bf16 codes in the workspace, then the bf16 kernels with
    // per-row scales
    case KV_E4M3: return launch_prefill_bf16(p, ws, stream, true);
    default: return launch_prefill_bf16(p, ws, stream, false);
  }
}

}  // namespace hs2

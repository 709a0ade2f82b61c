// Sparse reuse attention (one sparse layer over the index set chosen by the
// full layer).  HySparse2 pages, agihunt.info summary, inner-level paragraph:
// the sparse layers reuse the K/V rows of the selected tokens, and the forced
// local window and the global picks are read from the same full-attention K/V.
//
//   o[q,h,:] = sum_{j in S_q} softmax_{j in S_q}(scale <q_h, k_j>) v_j
//
// Design (gfx950):
//  * one workgroup (4 waves) per query token; the selected set is cut into
//    steps of STEP keys dealt round-robin to the waves, each wave keeps an
//    online-softmax state, and the four states are merged through LDS at the
//    end (no atomics, deterministic);
//  * the H <= 16 query heads share every K/V row (MQA), so they form the N
//    axis of 16x16 MFMA tiles (attn_tile.hpp);
//  * K fragments go straight from HBM/L2 into registers (four lanes cover 64
//    contiguous bytes of a gathered row per load instruction); V rows are
//    staged row-major in LDS and read back transposed;
//  * e4m3 caches are widened to bf16 exactly in registers; the row scales
//    multiply the logits (K) and are folded into P (V).
#include "attn_tile.hpp"
#include "hs2_internal.hpp"

namespace hs2 {
namespace {

constexpr int SP_WAVES = 4;
constexpr int SP_THREADS = SP_WAVES * kWave;
constexpr int kSlotBytes = 3 * 32 * 4;
constexpr int kWaveBytes = kTileStageBytes + kSlotBytes;
constexpr int kRedPitch = 260;
constexpr int kRedBytes = (SP_WAVES * 16 * kRedPitch + 2 * SP_WAVES * 16) * 4;
constexpr int kSmemBytes = (SP_WAVES * kWaveBytes > kRedBytes) ? SP_WAVES * kWaveBytes : kRedBytes;

template <int KV, int H>
__global__ __launch_bounds__(SP_THREADS, 2) void sparse_attn_kernel(const SparseParams p) {
  constexpr int STEP = TileCfg<KV>::STEP;
  constexpr int NMT = STEP / 16;
  constexpr int ROWB = (KV == KV_F32) ? 1024 : (KV == KV_BF16 ? 512 : 256);
  __shared__ __attribute__((aligned(16))) char smem[kSmemBytes];

  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int g = l >> 4, c16 = l & 15;
  const int qid = xcd_remap(blockIdx.x, gridDim.x);
  const int b = qid / p.n_q;
  const int64_t T = p.T;

  char* stage = smem + wave * kWaveBytes;
  int* s_key = (int*)(stage + kTileStageBytes);
  float* s_ksc = (float*)(s_key + 32);
  float* s_vsc = s_ksc + 32;

  QFrag qf;
  load_qfrag<KV>((const char*)p.q + ((int64_t)qid * H + c16) * kHeadDim * (KV == KV_F32 ? 4 : 2), c16 < H, g, qf);

  const int nsel = min(max(p.count[qid], 0), p.max_sel);
  const int nsteps = (nsel + STEP - 1) / STEP;
  const int32_t* irow = p.idx + (int64_t)qid * p.max_sel;
  const int64_t kv_row0 = (int64_t)b * T;
  const char* kseq = (const char*)p.k + kv_row0 * ROWB;
  const char* vseq = (const char*)p.v + kv_row0 * ROWB;

  float m_run = kNegInf, z_run = 0.f;
  f32x4 oacc[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) oacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int st = wave; st < nsteps; st += SP_WAVES) {
    // ---- slot table of this step (key index or -1, scales)
    if (l < STEP) {
      const int pos = st * STEP + l;
      int key = -1;
      if (pos < nsel) {
        const int j = irow[pos];
        if (j >= 0 && (int64_t)j < T) key = j;
      }
      s_key[l] = key;
      if constexpr (KV == KV_E4M3) {
        s_ksc[l] = key >= 0 ? p.k_scale[kv_row0 + key] : 0.f;
        s_vsc[l] = key >= 0 ? p.v_scale[kv_row0 + key] : 0.f;
      }
    }
    wave_lds_order();

    f32x4 sacc[NMT];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      const int key = s_key[16 * mt + c16];
      sacc[mt] = s_tile<KV>(key >= 0 ? kseq + (int64_t)key * ROWB : nullptr, g, qf);
    }
    stage_v<KV>(stage, l, [&](int slot) -> const char* {
      const int key = s_key[slot];
      return key >= 0 ? vseq + (int64_t)key * ROWB : nullptr;
    });

    // ---- online softmax (log2 domain); lane: row c16, key slots 16mt + 4g + r
    float x[NMT][4];
    float tmax = kNegInf;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int slot = 16 * mt + 4 * g + r;
        float v = sacc[mt][r] * p.scale_log2;
        if constexpr (KV == KV_E4M3) v *= s_ksc[slot];
        v = s_key[slot] >= 0 ? v : kNegInf;
        x[mt][r] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = fmaxf(tmax, shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m_run - m_new);
    float pr[NMT][4];
    float psum = 0.f;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = (x[mt][r] == kNegInf) ? 0.f : fast_exp2(x[mt][r] - m_new);
        psum += e;
        pr[mt][r] = e;
        if constexpr (KV == KV_E4M3) pr[mt][r] = e * s_vsc[16 * mt + 4 * g + r];
      }
    z_run = z_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int t = 0; t < 16; ++t) oacc[t] *= alpha;

    wave_lds_order();
    pv_step<KV>(stage, pr, g, c16, oacc);
    wave_lds_order();
  }

  // ---- merge: lane groups share the running max, their partial sums add up
  z_run += shfl_xor(z_run, 16);
  z_run += shfl_xor(z_run, 32);
  __syncthreads();
  float* red_o = (float*)smem;
  float* red_m = red_o + SP_WAVES * 16 * kRedPitch;
  float* red_z = red_m + SP_WAVES * 16;
  if (l < 16) {
    red_m[wave * 16 + l] = m_run;
    red_z[wave * 16 + l] = z_run;
  }
#pragma unroll
  for (int t = 0; t < 16; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) red_o[(wave * 16 + c16) * kRedPitch + 16 * t + 4 * g + r] = oacc[t][r];
  __syncthreads();

  for (int e = tid; e < H * kHeadDim; e += SP_THREADS) {
    const int h = e / kHeadDim, d = e % kHeadDim;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < SP_WAVES; ++w) M = fmaxf(M, red_m[w * 16 + h]);
    float Z = 0.f, acc = 0.f;
#pragma unroll
    for (int w = 0; w < SP_WAVES; ++w) {
      const float mw = red_m[w * 16 + h];
      if (mw != kNegInf) {
        const float f = fast_exp2(mw - M);
        Z += red_z[w * 16 + h] * f;
        acc += red_o[(w * 16 + h) * kRedPitch + d] * f;
      }
    }
    const float out = Z > 0.f ? acc / Z : 0.f;
    const int64_t oi = ((int64_t)qid * H + h) * kHeadDim + d;
    if constexpr (KV == KV_F32)
      ((float*)p.o)[oi] = out;
    else
      ((bf16*)p.o)[oi] = to_bf16(out);
    if (d == 0 && p.lse) p.lse[(int64_t)qid * H + h] = Z > 0.f ? (M + fast_log2(Z)) * kLn2 : kNegInf;
  }
}

template <int KV>
hipError_t launch_kv(const SparseParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)(p.B * p.n_q)), block(SP_THREADS);
  switch (p.H) {
    case 1: hipLaunchKernelGGL((sparse_attn_kernel<KV, 1>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((sparse_attn_kernel<KV, 2>), grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL((sparse_attn_kernel<KV, 4>), grid, block, 0, stream, p); break;
    case 8: hipLaunchKernelGGL((sparse_attn_kernel<KV, 8>), grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL((sparse_attn_kernel<KV, 16>), grid, block, 0, stream, p); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_attn(const SparseParams& p, int /*q_kind*/, int kv_kind, hipStream_t stream) {
  if (p.B * p.n_q == 0) return hipSuccess;
  switch (kv_kind) {
    case KV_F32: return launch_kv<KV_F32>(p, stream);
    case KV_BF16: return launch_kv<KV_BF16>(p, stream);
    default: return launch_kv<KV_E4M3>(p, stream);
  }
}

}  // namespace hs2

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
//  * K and V rows are gathered whole (each load instruction covers two bf16
//    or four e4m3 rows), then pass through the wave's LDS stage: K read back
//    as MFMA fragments, then V, row-major, read back transposed.  Loaded
//    straight into the fragment layout, a K load instruction would cover 16
//    rows x 64 B and request every cache line twice;
//  * e4m3 caches are widened to bf16 exactly in registers; the row scales
//    multiply the logits (K) and are folded into P (V);
//  * few queries (decode: B * n_q <= 64) would leave most CUs idle, so their
//    selected sets are also split into 128-key pieces, one workgroup each,
//    whose partial states (max, sum, unnormalised O) a second kernel merges.
#include <mutex>

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

constexpr int SP_SPLIT_KEYS = 128;   // selected keys per workgroup in the split form
constexpr int SP_SPLIT_MAXQ = 64;     // queries (B * n_q) up to which the set is split
constexpr int SP_MAX_PIECES = (kMaxSelect + SP_SPLIT_KEYS - 1) / SP_SPLIT_KEYS;   // pieces of the largest set

struct SparseWs {
  float* m;   // [B*n_q][nsplit][16]
  float* z;   // [B*n_q][nsplit][16]
  float* o;   // [B*n_q][nsplit][16][256]
  int nsplit;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// layout of the split workspace (base may be null: sizes only)
size_t sparse_ws_layout(int B, int n_q, int max_sel, char* base, SparseWs* ws) {
  const int64_t nq = (int64_t)B * n_q;
  if (nq > SP_SPLIT_MAXQ) {
    if (ws) *ws = SparseWs{nullptr, nullptr, nullptr, 1};
    return 0;
  }
  const int nsplit = (max_sel + SP_SPLIT_KEYS - 1) / SP_SPLIT_KEYS;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* ptr = base ? base + off : nullptr;
    off += align256(bytes);
    return (float*)ptr;
  };
  SparseWs w;
  w.m = take((size_t)nq * nsplit * 16 * 4);
  w.z = take((size_t)nq * nsplit * 16 * 4);
  w.o = take((size_t)nq * nsplit * 16 * kHeadDim * 4);
  w.nsplit = nsplit;
  if (ws) *ws = w;
  return off;
}

template <int KV, int H, bool SPLIT>
__global__ __launch_bounds__(SP_THREADS, 2) void sparse_attn_kernel(const SparseParams p, const SparseWs ws) {
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
  int* tab = (int*)(stage + kTileStageBytes);  // key of each slot of the step, or -1
  float* tks = (float*)(tab + 32);             // K row scales (e4m3)
  float* tvs = tks + 32;                       // V row scales (e4m3)

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

  // split form: this workgroup takes the steps of keys [split * 128, split * 128 + 128)
  const int split = SPLIT ? (int)blockIdx.y : 0;
  const int st_first = SPLIT ? split * (SP_SPLIT_KEYS / STEP) : 0;
  const int st_end = SPLIT ? min(nsteps, st_first + SP_SPLIT_KEYS / STEP) : nsteps;

  // Each step of a wave has one gather latency on its path: the index
  // entries of the next step are read while this one computes, and the K
  // rows, V rows (and scales) of a step are all issued together before the
  // first of them is waited for.  An absent key (past the count, or an index
  // outside [0, T)) reads row 0 and is masked out of the softmax, so every
  // load is unconditional.  The float32 cache loads V after the logits: its
  // K and V fragments together would not fit in the registers.
  constexpr bool V_EARLY = KV != KV_F32;
  auto fetch_key = [&](int st) -> int {  // lanes < STEP: key of slot l of step st, or -1
    const int pos = st * STEP + l;
    const bool in = l < STEP && st < st_end && pos < nsel;
    const int j = irow[in ? pos : 0];
    return (in && j >= 0 && (int64_t)j < T) ? j : -1;
  };
  int st = st_first + wave;
  int key = fetch_key(st);
  for (; st < st_end; st += SP_WAVES) {
    if (l < STEP) tab[l] = key;
    wave_lds_order();
    float ksc = 0.f, vsc = 0.f;
    if constexpr (KV == KV_E4M3) {
      ksc = p.k_scale[kv_row0 + max(key, 0)];
      vsc = p.v_scale[kv_row0 + max(key, 0)];
    }
    u32x4 kr[NMT][FragRegs<KV>::K], vr[FragRegs<KV>::V];
    auto load_v = [&] { load_v_rows<KV, false>(l, [&](int slot) { return vseq + (int64_t)max(tab[slot], 0) * ROWB; }, vr); };
    if constexpr (KV == KV_F32) {
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) load_k_tile<KV>(kseq + (int64_t)max(tab[16 * mt + c16], 0) * ROWB, g, kr[mt]);
    } else {
      static_assert(NMT * FragRegs<KV>::K == FragRegs<KV>::V, "K rows fill the fragment registers");
      load_v_rows<KV, false>(l, [&](int slot) { return kseq + (int64_t)max(tab[slot], 0) * ROWB; }, &kr[0][0]);
    }
    if constexpr (V_EARLY) load_v();
    key = fetch_key(st + SP_WAVES);
    if constexpr (KV != KV_F32) {
      store_k_rows<KV>(stage, l, &kr[0][0]);
      wave_lds_order();
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) read_k_tile<KV>(stage, mt, c16, g, kr[mt]);
    }

    f32x4 sacc[NMT];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) sacc[mt] = s_from_k<KV>(kr[mt], qf);
    if constexpr (!V_EARLY) load_v();
    store_v_rows<KV>(stage, l, vr);
    if constexpr (KV == KV_E4M3) {
      if (l < STEP) {
        tks[l] = ksc;
        tvs[l] = vsc;
      }
    }
    wave_lds_order();

    // ---- online softmax (log2 domain); lane: row c16, key slots 16mt + 4g + r
    float x[NMT][4];
    float tmax = kNegInf;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int slot = 16 * mt + 4 * g + r;
        float v = sacc[mt][r] * p.scale_log2;
        if constexpr (KV == KV_E4M3) v *= tks[slot];
        v = tab[slot] >= 0 ? v : kNegInf;
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
        if constexpr (KV == KV_E4M3) pr[mt][r] = e * tvs[16 * mt + 4 * g + r];
      }
    z_run = z_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int t = 0; t < 16; ++t) oacc[t] *= alpha;

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
    if constexpr (SPLIT) {
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
      const int64_t pi = ((int64_t)qid * ws.nsplit + split) * 16 + h;
      ws.o[pi * kHeadDim + d] = acc;
      if (d == 0) {
        ws.m[pi] = M;
        ws.z[pi] = Z;
      }
      continue;
    }
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

// Merge of the split partial states: workgroup (query, head), thread = dim.
template <int QKIND>
__global__ __launch_bounds__(256) void sparse_merge_kernel(const SparseParams p, const SparseWs ws) {
  const int qid = blockIdx.x, h = blockIdx.y, d = threadIdx.x;
  const int64_t b0 = (int64_t)qid * ws.nsplit * 16 + h;
  // every piece's (max, sum, O) is loaded up front (indices past the last
  // piece repeat it and are masked), so the merge costs one memory latency
  float mc[SP_MAX_PIECES], zc[SP_MAX_PIECES], oc[SP_MAX_PIECES];
#pragma unroll
  for (int i = 0; i < SP_MAX_PIECES; ++i) {
    const int64_t c = b0 + (int64_t)min(i, ws.nsplit - 1) * 16;
    mc[i] = ws.m[c];
    zc[i] = ws.z[c];
    oc[i] = ws.o[c * kHeadDim + d];
  }
  float M = kNegInf;
#pragma unroll
  for (int i = 0; i < SP_MAX_PIECES; ++i) {
    if (i >= ws.nsplit) mc[i] = kNegInf;
    M = fmaxf(M, mc[i]);
  }
  float Z = 0.f, acc = 0.f;
  // a piece without keys is masked by a select (its z and o may hold any bits)
#pragma unroll
  for (int i = 0; i < SP_MAX_PIECES; ++i) {
    const bool ok = mc[i] != kNegInf;
    const float f = fast_exp2(mc[i] - M);
    Z += ok ? zc[i] * f : 0.f;
    acc += ok ? oc[i] * f : 0.f;
  }
  const float out = Z > 0.f ? acc / Z : 0.f;
  const int64_t oi = ((int64_t)qid * gridDim.y + h) * kHeadDim + d;
  if constexpr (QKIND == KV_F32)
    ((float*)p.o)[oi] = out;
  else
    ((bf16*)p.o)[oi] = to_bf16(out);
  if (d == 0 && p.lse) p.lse[(int64_t)qid * gridDim.y + h] = Z > 0.f ? (M + fast_log2(Z)) * kLn2 : kNegInf;
}

template <int KV, int H>
void launch_h(const SparseParams& p, const SparseWs& ws, bool split, hipStream_t stream) {
  const unsigned nq = (unsigned)(p.B * p.n_q);
  if (split) {
    hipLaunchKernelGGL((sparse_attn_kernel<KV, H, true>), dim3(nq, ws.nsplit), dim3(SP_THREADS), 0, stream, p, ws);
    hipLaunchKernelGGL((sparse_merge_kernel<KV == KV_F32 ? KV_F32 : KV_BF16>), dim3(nq, H), dim3(256), 0, stream, p, ws);
  } else {
    hipLaunchKernelGGL((sparse_attn_kernel<KV, H, false>), dim3(nq), dim3(SP_THREADS), 0, stream, p, ws);
  }
}

template <int KV>
hipError_t launch_kv(const SparseParams& p, const SparseWs& ws, bool split, hipStream_t stream) {
  switch (p.H) {
    case 1: launch_h<KV, 1>(p, ws, split, stream); break;
    case 2: launch_h<KV, 2>(p, ws, split, stream); break;
    case 4: launch_h<KV, 4>(p, ws, split, stream); break;
    case 8: launch_h<KV, 8>(p, ws, split, stream); break;
    default: launch_h<KV, 16>(p, ws, split, stream); break;
  }
  return hipGetLastError();
}

// ---- scratch of the allocation-free entry point -------------------------
// The split form's partial states for at most kSparseStaticPieces (query,
// 128-key piece) pairs live in this file-scope device array (each GPU the
// library runs on holds its own copy until the process ends).  Host code never
// uses the array's name as an address: the device address comes from
// hipGetSymbolAddress, once per device, and is passed to the kernels like a
// workspace.  Nothing in it needs to start at zero (every piece writes its own
// slots before the merge reads them).
constexpr size_t kSparseStaticBytes = sparse_static_bytes();
static __device__ __align__(256) char scratch[kSparseStaticBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// device address of `scratch` on the current device
hipError_t static_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

size_t sparse_workspace_bytes(int B, int n_q, int max_sel) { return sparse_ws_layout(B, n_q, max_sel, nullptr, nullptr); }

hipError_t launch_sparse_attn_static(const SparseParams& p, int q_kind, int kv_kind, hipStream_t stream) {
  void* ws = nullptr;
  if (sparse_workspace_bytes(p.B, p.n_q, p.max_sel) > 0) {
    const hipError_t e = static_scratch(&ws);
    if (e != hipSuccess) return e;
  }
  return launch_sparse_attn(p, q_kind, kv_kind, ws, stream);
}

hipError_t launch_sparse_attn(const SparseParams& p, int /*q_kind*/, int kv_kind, void* ws_ptr, hipStream_t stream) {
  if (p.B * p.n_q == 0) return hipSuccess;
  SparseWs ws;
  const bool split = sparse_ws_layout(p.B, p.n_q, p.max_sel, (char*)ws_ptr, &ws) > 0;
  switch (kv_kind) {
    case KV_F32: return launch_kv<KV_F32>(p, ws, split, stream);
    case KV_BF16: return launch_kv<KV_BF16>(p, ws, split, stream);
    default: return launch_kv<KV_E4M3>(p, ws, split, stream);
  }
}

}  // namespace hs2

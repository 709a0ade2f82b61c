// Scored full attention, few-query path (decode: n_q * H <= 16 rows).
//
// Same definition as the prefill path (HySparse2 pages, agihunt.info summary:
// the full layer's exact attention probabilities score the tokens for the
// sparse layers), computed as a split over keys because one decode row has
// little work per key and the K/V stream (512 MiB at 1M FP8 tokens) must run
// at HBM speed:
//   split        : grid (key chunks, sequences); each workgroup computes the
//                  float32 logits of its keys (kept in the workspace, log2
//                  units), and a partial softmax state (max, sum, unnormalised
//                  O) per row;
//   merge        : while more than 32 states per row are left, a tree level of
//                  workgroups merges them, 32 at a time;
//   merge+score  : one launch finishes: some workgroups merge the last states
//                  into O and lse, the others derive the final lse of every row
//                  from the same states and write the scores of a key range,
//                  s_j = sum_h exp2(x_hj - lse2_h).
// No atomics: every partial has its own slot, so results are deterministic.
#include "attn_tile.hpp"
#include "hs2_internal.hpp"

namespace hs2 {
namespace {

constexpr int DC_WAVES = 4;
constexpr int DC_THREADS = DC_WAVES * kWave;
constexpr int kRedPitch = 260;
constexpr int kDcSmem = (DC_WAVES * kTileStageBytes > (DC_WAVES * 16 * kRedPitch + 2 * DC_WAVES * 16) * 4)
                            ? DC_WAVES * kTileStageBytes
                            : (DC_WAVES * 16 * kRedPitch + 2 * DC_WAVES * 16) * 4;

struct DecodeWs {
  float* logits;  // [B][T][16]  log2-domain logits of each row
  float* part_m;  // [B][nch][16]
  float* part_z;  // [B][nch][16]
  float* part_o;  // [B][nch][16][256]
  float* mid_m;   // [B][nmid][16]       partial states after one merge level
  float* mid_z;   // [B][nmid][16]
  float* mid_o;   // [B][nmid][16][256]
  int chunk, nch, nmid;
};
constexpr int kMergeFan = 32;   // partial states merged per workgroup and level

int decode_chunk(int B, int64_t T) {
  const int64_t total = (int64_t)B * T;
  int ch = 256;
  while (ch < 8192 && total / ch > 512) ch *= 2;   // about two workgroups per CU
  return ch;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t decode_ws_layout(int B, int64_t T, char* base, DecodeWs* ws) {
  const int ch = decode_chunk(B, T);
  const int64_t nch = (T + ch - 1) / ch;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* ptr = base ? base + off : nullptr;
    off += align256(bytes);
    return (float*)ptr;
  };
  DecodeWs w;
  w.logits = take((size_t)B * T * 16 * 4);
  w.part_m = take((size_t)B * nch * 16 * 4);
  w.part_z = take((size_t)B * nch * 16 * 4);
  w.part_o = take((size_t)B * nch * 16 * 256 * 4);
  const int64_t nmid = (nch + kMergeFan - 1) / kMergeFan;
  w.mid_m = take((size_t)B * nmid * 16 * 4);
  w.mid_z = take((size_t)B * nmid * 16 * 4);
  w.mid_o = take((size_t)B * nmid * 16 * 256 * 4);
  w.chunk = ch;
  w.nch = (int)nch;
  w.nmid = (int)nmid;
  if (ws) *ws = w;
  return off;
}

template <int KV, int H>
__global__ __launch_bounds__(DC_THREADS, 2) void decode_split_kernel(const AttnParams p, const DecodeWs ws) {
  constexpr int STEP = TileCfg<KV>::STEP;
  constexpr int NMT = STEP / 16;
  constexpr int ROWB = (KV == KV_F32) ? 1024 : (KV == KV_BF16 ? 512 : 256);
  constexpr int QB = (KV == KV_F32) ? 4 : 2;
  __shared__ __attribute__((aligned(16))) char smem[kDcSmem];

  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int g = l >> 4, c16 = l & 15;
  const int chunk = blockIdx.x, b = blockIdx.y;
  const int R = p.n_q * H;
  const bool row_ok = c16 < R;
  const int64_t row_pos = row_ok ? p.q_pos0 + c16 / H : -1;
  const int64_t n_keys = p.q_pos0 + p.n_q;
  const int64_t key0 = (int64_t)chunk * ws.chunk;
  const int64_t key1 = min(n_keys, key0 + ws.chunk);
  const int64_t kv_row0 = (int64_t)b * p.T;
  const char* kseq = (const char*)p.k + kv_row0 * ROWB;
  const char* vseq = (const char*)p.v + kv_row0 * ROWB;
  float* lg = ws.logits + kv_row0 * 16;
  char* stage = smem + wave * kTileStageBytes;

  QFrag qf;
  load_qfrag<KV>((const char*)p.q + ((int64_t)b * R + c16) * kHeadDim * QB, row_ok, g, qf);

  float m_run = kNegInf, z_run = 0.f;
  f32x4 oacc[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) oacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nst = (int)((key1 - key0 + STEP - 1) / STEP);
  for (int st = wave; st < nst; st += DC_WAVES) {
    const int64_t kb = key0 + (int64_t)st * STEP;
    f32x4 sacc[NMT];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      const int64_t key = kb + 16 * mt + c16;
      sacc[mt] = s_tile<KV>(key < key1 ? kseq + key * ROWB : nullptr, g, qf);
    }
    stage_v<KV>(stage, l, [&](int slot) -> const char* {
      const int64_t key = kb + slot;
      return key < key1 ? vseq + key * ROWB : nullptr;
    });
    float x[NMT][4];
    float tmax = kNegInf;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t key = kb + 16 * mt + 4 * g + r;
        float v = sacc[mt][r] * p.scale_log2;
        if constexpr (KV == KV_E4M3) v *= (key < key1) ? p.k_scale[kv_row0 + key] : 0.f;
        v = (key < key1 && key <= row_pos) ? v : kNegInf;
        if (row_ok && key < key1) lg[key * 16 + c16] = v;
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
        if constexpr (KV == KV_E4M3) {
          const int64_t key = kb + 16 * mt + 4 * g + r;
          pr[mt][r] = (key < key1) ? e * p.v_scale[kv_row0 + key] : 0.f;
        }
      }
    z_run = z_run * alpha + psum;
    m_run = m_new;
    if (__any(alpha != 1.f)) {   // the running max rarely moves after the first steps
#pragma unroll
      for (int t = 0; t < 16; ++t) oacc[t] *= alpha;
    }
    wave_lds_order();
    pv_step<KV>(stage, pr, g, c16, oacc);
    wave_lds_order();
  }

  // ---- merge the 4 lane groups and 4 waves into this chunk's partial state
  z_run += shfl_xor(z_run, 16);
  z_run += shfl_xor(z_run, 32);
  __syncthreads();
  float* red_o = (float*)smem;
  float* red_m = red_o + DC_WAVES * 16 * kRedPitch;
  float* red_z = red_m + DC_WAVES * 16;
  if (l < 16) {
    red_m[wave * 16 + l] = m_run;
    red_z[wave * 16 + l] = z_run;
  }
#pragma unroll
  for (int t = 0; t < 16; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) red_o[(wave * 16 + c16) * kRedPitch + 16 * t + 4 * g + r] = oacc[t][r];
  __syncthreads();
  const int64_t pbase = ((int64_t)b * ws.nch + chunk) * 16;
  for (int e = tid; e < R * kHeadDim; e += DC_THREADS) {
    const int row = e / kHeadDim, d = e % kHeadDim;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < DC_WAVES; ++w) M = fmaxf(M, red_m[w * 16 + row]);
    float Z = 0.f, acc = 0.f;
#pragma unroll
    for (int w = 0; w < DC_WAVES; ++w) {
      const float mw = red_m[w * 16 + row];
      if (mw != kNegInf) {
        const float f = fast_exp2(mw - M);
        Z += red_z[w * 16 + row] * f;
        acc += red_o[(w * 16 + row) * kRedPitch + d] * f;
      }
    }
    ws.part_o[(pbase + row) * kHeadDim + d] = acc;
    if (d == 0) {
      ws.part_m[pbase + row] = M;
      ws.part_z[pbase + row] = Z;
    }
  }
}

// bf16 / e4m3 caches: the 4 waves of a workgroup take turns over the chunk's
// 16-key steps (together they stream one contiguous range), and each wave
// keeps its next step's K and V rows in flight (registers) while the current
// step is computed, so that every wave always has about 16 KB of HBM reads
// outstanding.  S^T (16 keys x 16 rows) is 8 MFMAs
// 16x16x32 with K straight from the registers; V goes through a wave-private
// LDS tile and feeds O^T += V^T P^T as 16 MFMAs 16x16x16 (A = V^T by
// transposed reads, B = P^T straight from the S^T layout).
constexpr int DS_STEP = 16;
constexpr int DS_VPITCH = 272;                       // bf16 elements per staged V row (544 B)
constexpr int DS_VTILE = DS_STEP * DS_VPITCH * 2;    // 8704 B per wave
constexpr int DS_RED = (DC_WAVES * 16 * kRedPitch + 2 * DC_WAVES * 16) * 4;
constexpr int DS_LGT = DS_STEP * 16 * 4;               // 1 KB: one step's logits [key][row] per wave
constexpr int DS_LOOP = DC_WAVES * (DS_VTILE + DS_LGT);  // V tiles, then logits tiles
constexpr int DS_SMEM = DS_LOOP > DS_RED ? DS_LOOP : DS_RED;

template <int KV>
struct DsRegs {
  static constexpr int NK = KV == KV_BF16 ? 8 : 4;   // 16-byte K pieces per lane
  u32x4 k[NK];
  float ks[4], vs[4];                                // e4m3 row scales of keys kb + 4g + i
};
template <int KV>
struct DsVRegs {
  static constexpr int NV = KV == KV_BF16 ? 8 : 4;   // 16-byte V pieces per lane
  u32x4 v[NV];
};

typedef short i16x4_t __attribute__((ext_vector_type(4)));

template <int KV, int H>
__global__ __launch_bounds__(DC_THREADS, 2) void decode_stream_kernel(const AttnParams p, const DecodeWs ws) {
  constexpr int ROWB = (KV == KV_BF16) ? 512 : 256;
  __shared__ __attribute__((aligned(16))) char smem[DS_SMEM];

  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int g = l >> 4, c16 = l & 15;
  const int chunk = blockIdx.x, b = blockIdx.y;
  const int R = p.n_q * H;
  const bool row_ok = c16 < R;
  const int64_t row_pos = row_ok ? p.q_pos0 + c16 / H : -1;
  const int64_t n_keys = p.q_pos0 + p.n_q;
  const int64_t key0 = (int64_t)chunk * ws.chunk;
  const int64_t key1 = min(n_keys, key0 + ws.chunk);
  // the 4 waves interleave 16-key steps: together they stream one contiguous range
  const int wvu = __builtin_amdgcn_readfirstlane(wave);
  const int64_t kw0 = key0 + wvu * DS_STEP;               // first key of this wave's first step
  const int64_t kw1 = key1;
  const int nst_all = key1 > key0 ? (int)((key1 - key0 + DS_STEP - 1) / DS_STEP) : 0;
  const int nst = nst_all > wvu ? (nst_all - wvu + DC_WAVES - 1) / DC_WAVES : 0;
  const int64_t kv_row0 = (int64_t)b * p.T;
  const char* kseq = (const char*)p.k + kv_row0 * ROWB;
  const char* vseq = (const char*)p.v + kv_row0 * ROWB;
  float* lg = ws.logits + kv_row0 * 16;
  bf16* vt = (bf16*)(smem + wave * DS_VTILE);
  float* lgt = (float*)(smem + DC_WAVES * DS_VTILE + wave * DS_LGT);

  QFrag qf;
  load_qfrag<KV>((const char*)p.q + ((int64_t)b * R + c16) * kHeadDim * 2, row_ok, g, qf);

  // ---- loads of step st: K of key kb + c16 (the lane's MFMA row) and the
  // e4m3 scales of keys kb + 4g + i
  // Keys past the wave's range load its last row instead (no branches around
  // the loads, so the compiler can count them): their logits are masked and
  // their probabilities are zero.  The K/V stream is read once: nontemporal
  // loads (measured on an MI355X: 6.2-6.9 TB/s for a plain stream against
  // 4.4 TB/s with ordinary loads).
  // V: each load instruction reads whole rows (bf16: two rows of 512 B, e4m3:
  // four rows of 256 B), so that every cache line is requested once
  constexpr int VRPI = 1024 / ROWB;   // rows per load instruction
  auto load_v = [&](int st, DsVRegs<KV>& r) __attribute__((always_inline)) {
    const int64_t kb = kw0 + (int64_t)st * (DS_STEP * DC_WAVES);
#pragma unroll
    for (int j = 0; j < DsVRegs<KV>::NV; ++j) {
      const int64_t kv = min(kb + VRPI * j + l / (64 / VRPI), kw1 - 1);
      r.v[j] = ld_nt((const u32x4*)(vseq + kv * ROWB + 16 * (l % (64 / VRPI))));
    }
  };
  auto load_k = [&](int st, DsRegs<KV>& r) __attribute__((always_inline)) {
    const int64_t kb = kw0 + (int64_t)st * (DS_STEP * DC_WAVES);
    const int64_t kk = min(kb + c16, kw1 - 1);
    const char* kp = kseq + kk * ROWB;
#pragma unroll
    for (int j = 0; j < DsRegs<KV>::NK; ++j) {
      const int off = (KV == KV_BF16) ? (32 * j + 8 * g) * 2 : 64 * j + 16 * g;
      r.k[j] = ld_nt((const u32x4*)(kp + off));
    }
    if constexpr (KV == KV_E4M3) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t key = min(kb + 4 * g + i, kw1 - 1);
        r.ks[i] = p.k_scale[kv_row0 + key];
        r.vs[i] = p.v_scale[kv_row0 + key];
      }
    }
  };
  // Logits of the wave's keys through a buffer resource that ends at its last
  // key: stores past it are dropped (rows >= R hold unused slots).  A lane
  // holds 4 keys of one row; written as they are, every 128-byte line of the
  // [key][16] layout would be half-written by two store instructions, which
  // cost a plain K/V stream a quarter of its rate on the box (80 -> 108 us at
  // 16 x 32k keys).  So a step's 16 x 16 logits go through the wave's 1 KB LDS
  // tile and out as one contiguous 16-byte-per-lane store.
  const __amdgpu_buffer_rsrc_t lg_rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(lg + key0 * 16), 0, (int)(max((int64_t)0, key1 - key0) * 64), 0x00020000);
  // V rows of the step -> the wave's LDS tile (bf16, row pitch DS_VPITCH)
  auto stage = [&](const DsVRegs<KV>& r) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < DsVRegs<KV>::NV; ++j) {
      bf16* row = vt + (VRPI * j + l / (64 / VRPI)) * DS_VPITCH;
      if constexpr (KV == KV_BF16) {
        *(u32x4*)(row + 8 * (l % 32)) = r.v[j];
      } else {
        bf16* dst = row + 16 * (l % 16);
        *(bf16x8*)dst = e4m3x8_to_bf16(r.v[j][0], r.v[j][1]);
        *(bf16x8*)(dst + 8) = e4m3x8_to_bf16(r.v[j][2], r.v[j][3]);
      }
    }
  };

  float m_run = kNegInf, z_run = 0.f;   // z_run: this lane's keys only (summed over g at the end)
  f32x4 oacc[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) oacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int st, const DsRegs<KV>& r) __attribute__((always_inline)) {
    const int64_t kb = kw0 + (int64_t)st * (DS_STEP * DC_WAVES);
    // S^T: lane holds keys kb + 4g + i of row c16
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (KV == KV_BF16) {
#pragma unroll
      for (int j = 0; j < 8; ++j) acc = mfma16(as_bf16x8(r.k[j]), qf.b[j], acc);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc = mfma16(e4m3x8_to_bf16(r.k[j][0], r.k[j][1]), qf.b[2 * j], acc);
        acc = mfma16(e4m3x8_to_bf16(r.k[j][2], r.k[j][3]), qf.b[2 * j + 1], acc);
      }
    }
    float x[4];
    float tmax = kNegInf;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t key = kb + 4 * g + i;
      float v = acc[i] * p.scale_log2;
      if constexpr (KV == KV_E4M3) v *= r.ks[i];
      v = (key < kw1 && key <= row_pos) ? v : kNegInf;
      lgt[(4 * g + i) * 16 + c16] = v;
      x[i] = v;
      tmax = fmaxf(tmax, v);
    }
    // the wave's own tile: LDS keeps its writes and this read in order
    const u32x4 lg4 = *(const u32x4*)(lgt + 4 * l);
    __builtin_amdgcn_raw_buffer_store_b128(lg4, lg_rs, (int)((kb - key0) * 64 + 16 * l), 0, 0);
    tmax = fmaxf(tmax, shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m_run - m_new);
    bf16x4 pb;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float e = (x[i] == kNegInf) ? 0.f : fast_exp2(x[i] - m_new);
      psum += e;
      if constexpr (KV == KV_E4M3) e *= r.vs[i];   // finite: the clamped key's scale
      pb[i] = to_bf16(e);
    }
    z_run = z_run * alpha + psum;
    m_run = m_new;
    if (__any(alpha != 1.f)) {   // the running max rarely moves after the first steps
#pragma unroll
      for (int t = 0; t < 16; ++t) oacc[t] *= alpha;
    }
    // O^T += V^T P^T: A lane = column 16t + c16 of the tile rows 4g..4g+3
    const bf16* vr = vt + (4 * g + (c16 >> 2)) * DS_VPITCH + 4 * (c16 & 3);
    const i16x4_t pbi = __builtin_bit_cast(i16x4_t, pb);
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const i16x4_t a = __builtin_bit_cast(i16x4_t, lds_tr16(vr + 16 * t));
      oacc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pbi, oacc[t], 0, 0, 0);
    }
  };

  // K (and the scales) double-buffered in registers; the one set of V
  // registers is refilled with the next step's rows as soon as they are in LDS.
  // (Deeper buffering -- two V sets, or three K sets and two V sets with e4m3
  // rows -- measured no faster: the steady state already streams at about
  // 6.4 TB/s; the time above that goes to the first step's fill and to the
  // spread of the waves' finishing times.)
  DsRegs<KV> r0, r1;
  DsVRegs<KV> vr;
  if (nst > 0) {
    load_k(0, r0);
    load_v(0, vr);
  }
  for (int st = 0; st < nst; st += 2) {
    if (st + 1 < nst) load_k(st + 1, r1);
    stage(vr);
    if (st + 1 < nst) load_v(st + 1, vr);
    compute(st, r0);
    if (st + 1 < nst) {
      if (st + 2 < nst) load_k(st + 2, r0);
      stage(vr);
      if (st + 2 < nst) load_v(st + 2, vr);
      compute(st + 1, r1);
    }
  }

  // ---- merge the 4 lane groups and 4 waves into this chunk's partial state
  z_run += shfl_xor(z_run, 16);
  z_run += shfl_xor(z_run, 32);
  __syncthreads();
  float* red_o = (float*)smem;
  float* red_m = red_o + DC_WAVES * 16 * kRedPitch;
  float* red_z = red_m + DC_WAVES * 16;
  if (l < 16) {
    red_m[wave * 16 + l] = m_run;
    red_z[wave * 16 + l] = z_run;
  }
#pragma unroll
  for (int t = 0; t < 16; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) red_o[(wave * 16 + c16) * kRedPitch + 16 * t + 4 * g + r] = oacc[t][r];
  __syncthreads();
  const int64_t pbase = ((int64_t)b * ws.nch + chunk) * 16;
  for (int e = tid; e < R * kHeadDim; e += DC_THREADS) {
    const int row = e / kHeadDim, d = e % kHeadDim;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < DC_WAVES; ++w) M = fmaxf(M, red_m[w * 16 + row]);
    float Z = 0.f, acc = 0.f;
#pragma unroll
    for (int w = 0; w < DC_WAVES; ++w) {
      const float mw = red_m[w * 16 + row];
      if (mw != kNegInf) {
        const float f = fast_exp2(mw - M);
        Z += red_z[w * 16 + row] * f;
        acc += red_o[(w * 16 + row) * kRedPitch + d] * f;
      }
    }
    ws.part_o[(pbase + row) * kHeadDim + d] = acc;
    if (d == 0) {
      ws.part_m[pbase + row] = M;
      ws.part_z[pbase + row] = Z;
    }
  }
}

// One level of the merge of partial softmax states (m, z, unnormalised O)
// over key chunks: workgroup (g, row, b) merges the states g*F .. g*F+F-1 of
// one row (thread = head dim) into one state.  The order of the sums is
// fixed, so results are deterministic.
struct MergeIO {
  const float* in_m;
  const float* in_z;
  const float* in_o;
  float* out_m;
  float* out_z;
  float* out_o;
  int in_stride, nin, out_stride;   // states per sequence in the layouts; valid inputs
};

__global__ __launch_bounds__(256) void decode_merge_kernel(const AttnParams p, const DecodeWs ws, const MergeIO io) {
  const int g = blockIdx.x, row = blockIdx.y, b = blockIdx.z, d = threadIdx.x;
  const int c0 = g * kMergeFan, c1 = min(io.nin, c0 + kMergeFan);
  const int64_t ib = (int64_t)b * io.in_stride;
  // every load is issued up front (indices past the last state repeat it and
  // are masked), so the fan-in costs one memory latency, not one per state
  float mc[kMergeFan], zc[kMergeFan], oc[kMergeFan];
  float M = kNegInf;
#pragma unroll
  for (int i = 0; i < kMergeFan; ++i) {
    const int64_t c = ib + min(c0 + i, c1 - 1);
    mc[i] = io.in_m[c * 16 + row];
    zc[i] = io.in_z[c * 16 + row];
    oc[i] = io.in_o[(c * 16 + row) * kHeadDim + d];
  }
#pragma unroll
  for (int i = 0; i < kMergeFan; ++i) {
    if (c0 + i >= c1) mc[i] = kNegInf;
    M = fmaxf(M, mc[i]);
  }
  float Z = 0.f, acc = 0.f;
#pragma unroll
  for (int i = 0; i < kMergeFan; ++i) {
    const bool ok = mc[i] != kNegInf;   // a selected 0 adds exactly; masked terms may hold any bits
    const float f = fast_exp2(mc[i] - M);
    Z += ok ? zc[i] * f : 0.f;
    acc += ok ? oc[i] * f : 0.f;
  }
  const int64_t ob = ((int64_t)b * io.out_stride + g) * 16 + row;
  io.out_o[ob * kHeadDim + d] = acc;
  if (d == 0) {
    io.out_m[ob] = M;
    io.out_z[ob] = Z;
  }
}

// The last merge level and the scores in one launch (at most kMergeFan states
// per row are left).  Workgroups [0, B * R) merge the O of one (sequence, row)
// (thread = head dim, every load issued up front); the others score a range
// of keys after deriving the final lse of every row themselves from the same
// states' (max, sum) pairs, so no workgroup waits for another.  The sums run
// over the states in order: deterministic.
constexpr int MS_KEYS = 2048;   // keys scored per workgroup

template <int QKIND, int H>
__global__ __launch_bounds__(256) void decode_merge_score_kernel(const AttnParams p, const DecodeWs ws,
                                                                 const MergeIO io) {
  const int R = p.n_q * H;
  const int n_merge = p.B * R;
  const int tid = threadIdx.x;
  if ((int)blockIdx.x < n_merge) {
    const int b = blockIdx.x / R, row = blockIdx.x % R, d = tid;
    const int64_t ib = (int64_t)b * io.in_stride;
    float mc[kMergeFan], zc[kMergeFan], oc[kMergeFan];
    float M = kNegInf;
#pragma unroll
    for (int i = 0; i < kMergeFan; ++i) {
      const int64_t c = ib + min(i, io.nin - 1);
      mc[i] = io.in_m[c * 16 + row];
      zc[i] = io.in_z[c * 16 + row];
      oc[i] = io.in_o[(c * 16 + row) * kHeadDim + d];
    }
#pragma unroll
    for (int i = 0; i < kMergeFan; ++i) {
      if (i >= io.nin) mc[i] = kNegInf;
      M = fmaxf(M, mc[i]);
    }
    float Z = 0.f, acc = 0.f;
#pragma unroll
    for (int i = 0; i < kMergeFan; ++i) {
      const bool ok = mc[i] != kNegInf;   // a selected 0 adds exactly; masked terms may hold any bits
      const float f = fast_exp2(mc[i] - M);
      Z += ok ? zc[i] * f : 0.f;
      acc += ok ? oc[i] * f : 0.f;
    }
    const int64_t oi = ((int64_t)b * R + row) * kHeadDim + d;
    const float out = acc / Z;
    if constexpr (QKIND == KV_F32)
      ((float*)p.o)[oi] = out;
    else
      ((bf16*)p.o)[oi] = to_bf16(out);
    if (d == 0 && p.lse) p.lse[(int64_t)b * R + row] = (M + fast_log2(Z)) * kLn2;
    return;
  }
  // ---- scores of keys [key0, key0 + MS_KEYS) of one sequence
  const int64_t n_keys = p.q_pos0 + p.n_q;
  const int nblk = (int)((n_keys + MS_KEYS - 1) / MS_KEYS);
  const int sb = blockIdx.x - n_merge;
  const int b = sb / nblk;
  const int64_t key0 = (int64_t)(sb % nblk) * MS_KEYS;
  __shared__ float l2s[16];
  if (tid < 16) {
    float l2 = 0.f;
    if (tid < R) {
      const int64_t ib = (int64_t)b * io.in_stride;
      float mc[kMergeFan], zc[kMergeFan];
      float M = kNegInf;
#pragma unroll
      for (int i = 0; i < kMergeFan; ++i) {
        const int64_t c = ib + min(i, io.nin - 1);
        mc[i] = io.in_m[c * 16 + tid];
        zc[i] = io.in_z[c * 16 + tid];
      }
#pragma unroll
      for (int i = 0; i < kMergeFan; ++i) {
        if (i >= io.nin) mc[i] = kNegInf;
        M = fmaxf(M, mc[i]);
      }
      float Z = 0.f;
#pragma unroll
      for (int i = 0; i < kMergeFan; ++i) Z += mc[i] != kNegInf ? zc[i] * fast_exp2(mc[i] - M) : 0.f;
      l2 = M + fast_log2(Z);
    }
    l2s[tid] = l2;
  }
  __syncthreads();
  float l2[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) l2[r] = l2s[r];
  for (int64_t key = key0 + tid; key < min(n_keys, key0 + MS_KEYS); key += 256) {
    const float* x = ws.logits + ((int64_t)b * p.T + key) * 16;
    const f32x4 x0 = *(const f32x4*)x, x1 = *(const f32x4*)(x + 4), x2 = *(const f32x4*)(x + 8),
                x3 = *(const f32x4*)(x + 12);
    const float xs[16] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3],
                          x2[0], x2[1], x2[2], x2[3], x3[0], x3[1], x3[2], x3[3]};
    for (int i = 0; i < p.n_q; ++i) {
      if (key > p.q_pos0 + i) continue;
      float s = 0.f;
#pragma unroll
      for (int h = 0; h < H; ++h) s += fast_exp2(xs[(i * H + h) & 15] - l2[(i * H + h) & 15]);
      p.scores[((int64_t)b * p.n_q + i) * p.ld_scores + key] = s;
    }
  }
}

template <int KV, int H>
hipError_t launch_decode_h(const AttnParams& p, const DecodeWs& ws, hipStream_t stream) {
  const int64_t n_keys = p.q_pos0 + p.n_q;
  const unsigned nch = (unsigned)((n_keys + ws.chunk - 1) / ws.chunk);
  if constexpr (KV == KV_F32)
    hipLaunchKernelGGL((decode_split_kernel<KV, H>), dim3(nch, p.B), dim3(DC_THREADS), 0, stream, p, ws);
  else
    hipLaunchKernelGGL((decode_stream_kernel<KV, H>), dim3(nch, p.B), dim3(DC_THREADS), 0, stream, p, ws);
  const int R = p.n_q * p.H;
  // merge tree over the chunk states while more than kMergeFan are left:
  // part -> mid -> part -> ...; the last level and the scores share one launch
  MergeIO io{ws.part_m, ws.part_z, ws.part_o, ws.mid_m, ws.mid_z, ws.mid_o, ws.nch, (int)nch, ws.nmid};
  while (io.nin > kMergeFan) {
    const int nout = (io.nin + kMergeFan - 1) / kMergeFan;
    hipLaunchKernelGGL(decode_merge_kernel, dim3(nout, R, p.B), dim3(256), 0, stream, p, ws, io);
    const bool to_mid = io.out_m == ws.mid_m;
    io.in_m = io.out_m;
    io.in_z = io.out_z;
    io.in_o = io.out_o;
    io.in_stride = io.out_stride;
    io.nin = nout;
    io.out_m = to_mid ? ws.part_m : ws.mid_m;   // the inputs of the previous level are free again
    io.out_z = to_mid ? ws.part_z : ws.mid_z;
    io.out_o = to_mid ? ws.part_o : ws.mid_o;
    io.out_stride = to_mid ? ws.nch : ws.nmid;
  }
  const int nblk = (int)((n_keys + MS_KEYS - 1) / MS_KEYS);
  const dim3 grid((unsigned)(p.B * R + p.B * nblk));
  if (KV == KV_F32)
    hipLaunchKernelGGL((decode_merge_score_kernel<KV_F32, H>), grid, dim3(256), 0, stream, p, ws, io);
  else
    hipLaunchKernelGGL((decode_merge_score_kernel<KV_BF16, H>), grid, dim3(256), 0, stream, p, ws, io);
  return hipGetLastError();
}

template <int KV>
hipError_t launch_decode_kv(const AttnParams& p, const DecodeWs& ws, hipStream_t stream) {
  switch (p.H) {
    case 1: return launch_decode_h<KV, 1>(p, ws, stream);
    case 2: return launch_decode_h<KV, 2>(p, ws, stream);
    case 4: return launch_decode_h<KV, 4>(p, ws, stream);
    case 8: return launch_decode_h<KV, 8>(p, ws, stream);
    default: return launch_decode_h<KV, 16>(p, ws, stream);
  }
}

}  // namespace

hipError_t launch_prefill(const AttnParams& p, int kv_kind, void* ws, hipStream_t stream);  // attn_prefill.hip
size_t prefill_bf16_workspace_bytes(int B, int n_q, int H, int64_t T, bool e4m3);   // attn_prefill_bf16.hip

bool attn_uses_decode(int n_q, int H) { return (int64_t)n_q * H <= 16; }

size_t attn_workspace_bytes(int B, int n_q, int H, int64_t T, int kv_kind) {
  if (!attn_uses_decode(n_q, H))
    return kv_kind == KV_F32 ? 0 : prefill_bf16_workspace_bytes(B, n_q, H, T, kv_kind == KV_E4M3);
  return decode_ws_layout(B, T, nullptr, nullptr);
}

hipError_t launch_full_attn(const AttnParams& p, int /*q_kind*/, int kv_kind, void* ws_ptr, size_t /*ws_bytes*/,
                            hipStream_t stream) {
  if (p.B * p.n_q == 0) return hipSuccess;
  if (!attn_uses_decode(p.n_q, p.H)) return launch_prefill(p, kv_kind, ws_ptr, stream);
  DecodeWs ws;
  decode_ws_layout(p.B, p.T, (char*)ws_ptr, &ws);
  switch (kv_kind) {
    case KV_F32: return launch_decode_kv<KV_F32>(p, ws, stream);
    case KV_BF16: return launch_decode_kv<KV_BF16>(p, ws, stream);
    default: return launch_decode_kv<KV_E4M3>(p, ws, stream);
  }
}

}  // namespace hs2

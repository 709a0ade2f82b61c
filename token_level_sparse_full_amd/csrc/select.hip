// Token-level top-k with the forced recent window.  HySparse2 pages,
// agihunt.info summary, inner-level paragraph: block-level top-k becomes
// token-level, the separate SWA branch of the sparse layers is dropped, the
// 128 most recent tokens are always kept and the 1024 best-scoring tokens
// outside that window are added.  Ties in score go to the lower index (the
// reading taken here).
//
// For the query at position p: W = [p-window+1, p], C = [0, p-window].
// If |C| <= topk every key 0..p is selected.  Otherwise the topk-th largest
// candidate score tau is found exactly, and the selection is every candidate
// above tau plus the first (topk - #above) candidates equal to tau in index
// order, followed by the window; this is already ascending.
//
// Design: one 1024-thread workgroup per query row.  Scores are >= 0, so their
// float32 bit patterns order like unsigned integers.  A first pass finds the
// smallest and largest candidate pattern; the bits above their highest
// differing bit are common to all candidates, so the radix digits (11 bits,
// LDS histograms) start right below them and split the actual value range
// instead of the (nearly constant) exponent.  The compaction pass is a
// block-wide ordered scan that stops as soon as topk candidates are out.
#include "hs2_device.hpp"
#include "hs2_internal.hpp"

namespace hs2 {
namespace {

constexpr int SEL_THREADS = 1024;
constexpr int SEL_WAVES = SEL_THREADS / kWave;
constexpr int SEL_DIGIT = 11;
constexpr int SEL_BINS = 1 << SEL_DIGIT;

struct SelShared {
  int hist[SEL_BINS];
  int wave_tot[SEL_WAVES];
  uint32_t wave_u[2 * SEL_WAVES];
  int pick_digit;
  int pick_above;
};

__device__ __forceinline__ uint32_t fbits(float x) { return __builtin_bit_cast(uint32_t, x); }

// Inclusive scan of v over the wave.
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int t = __shfl_up(v, o, kWave);
    if (lane >= o) v += t;
  }
  return v;
}

// Exclusive block-wide scan; returns the exclusive prefix of v and the block total.
__device__ __forceinline__ int block_excl_scan(int v, int tid, SelShared& sh, int& total) {
  const int lane = tid & 63, wave = tid >> 6;
  const int inc = wave_incl_scan(v, lane);
  if (lane == 63) sh.wave_tot[wave] = inc;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < SEL_WAVES; ++w) {
    const int t = sh.wave_tot[w];
    before += (w < wave) ? t : 0;
    total += t;
  }
  __syncthreads();
  return before + inc - v;
}

__global__ __launch_bounds__(SEL_THREADS) void select_kernel(const SelectParams p) {
  __shared__ SelShared sh;
  const int tid = threadIdx.x;
  const int qid = xcd_remap(blockIdx.x, gridDim.x);
  const int i = qid % p.n_q;
  const int64_t pos = p.q_pos0 + i;
  const int64_t n = pos + 1;
  const int max_sel = p.window + p.topk;
  int32_t* out = p.idx + (int64_t)qid * max_sel;
  const float* row = p.scores + (int64_t)qid * p.ld_scores;
  const int64_t n_cand = n > p.window ? n - p.window : 0;

  if (n_cand <= p.topk) {  // every key 0..p is selected
    for (int j = tid; j < max_sel; j += SEL_THREADS) out[j] = j < n ? j : -1;
    if (tid == 0) p.count[qid] = (int32_t)n;
    return;
  }

  // ---- pass 0: smallest and largest candidate bit pattern
  uint32_t mx = 0u, mn = 0xFFFFFFFFu;
  const int64_t n4 = n_cand & ~(int64_t)3;
  for (int64_t j = 4 * (int64_t)tid; j < n4; j += 4 * SEL_THREADS) {
    const f32x4 v = *(const f32x4*)(row + j);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t u = fbits(v[e]);
      mx = max(mx, u);
      mn = min(mn, u);
    }
  }
  for (int64_t j = n4 + tid; j < n_cand; j += SEL_THREADS) {
    const uint32_t u = fbits(row[j]);
    mx = max(mx, u);
    mn = min(mn, u);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, o, kWave));
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, o, kWave));
  }
  if ((tid & 63) == 0) {
    sh.wave_u[tid >> 6] = mx;
    sh.wave_u[SEL_WAVES + (tid >> 6)] = mn;
  }
  __syncthreads();
  mx = 0u;
  mn = 0xFFFFFFFFu;
#pragma unroll
  for (int w = 0; w < SEL_WAVES; ++w) {
    mx = max(mx, sh.wave_u[w]);
    mn = min(mn, sh.wave_u[SEL_WAVES + w]);
  }

  // ---- radix passes below the common prefix
  uint32_t tau;
  int need_eq;  // how many candidates equal to tau are taken (in index order)
  if (mx == mn) {
    tau = mx;
    need_eq = p.topk;
  } else {
    const int hb = 31 - __builtin_clz(mx ^ mn);
    int shift = hb + 1;
    uint64_t prefix = (uint64_t)mx >> shift << shift;  // common high bits
    int krem = p.topk;
    while (shift > 0) {
      const int w = shift < SEL_DIGIT ? shift : SEL_DIGIT;
      shift -= w;
      const int nbins = 1 << w;
      const uint64_t want = prefix >> (shift + w);
      for (int b = tid; b < nbins; b += SEL_THREADS) sh.hist[b] = 0;
      __syncthreads();
      for (int64_t j = 4 * (int64_t)tid; j < n4; j += 4 * SEL_THREADS) {
        const f32x4 v = *(const f32x4*)(row + j);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint64_t u = fbits(v[e]);
          if ((u >> (shift + w)) == want) atomicAdd(&sh.hist[(u >> shift) & (nbins - 1)], 1);
        }
      }
      for (int64_t j = n4 + tid; j < n_cand; j += SEL_THREADS) {
        const uint64_t u = fbits(row[j]);
        if ((u >> (shift + w)) == want) atomicAdd(&sh.hist[(u >> shift) & (nbins - 1)], 1);
      }
      __syncthreads();
      // scan the bins from the top digit down; thread t owns digits nbins-1-2t, nbins-2-2t
      const int d0 = nbins - 1 - 2 * tid, d1 = d0 - 1;
      const int c0 = d0 >= 0 ? sh.hist[d0] : 0;
      const int c1 = d1 >= 0 ? sh.hist[d1] : 0;
      int total;
      const int before = block_excl_scan(c0 + c1, tid, sh, total);
      if (d0 >= 0) {
        if (before < krem && krem <= before + c0) {
          sh.pick_digit = d0;
          sh.pick_above = before;
        } else if (d1 >= 0 && before + c0 < krem && krem <= before + c0 + c1) {
          sh.pick_digit = d1;
          sh.pick_above = before + c0;
        }
      }
      __syncthreads();
      prefix |= (uint64_t)sh.pick_digit << shift;
      krem -= sh.pick_above;
      __syncthreads();
    }
    tau = (uint32_t)prefix;
    need_eq = krem;
  }

  // ---- ordered compaction: above tau, then the first need_eq ties
  int eq_seen = 0, sel_seen = 0;
  for (int64_t base = 0; base < n_cand && sel_seen < p.topk; base += 4 * SEL_THREADS) {
    const int64_t j0 = base + 4 * (int64_t)tid;
    uint32_t u[4];
    if (j0 + 3 < n_cand) {
      const f32x4 v = *(const f32x4*)(row + j0);
#pragma unroll
      for (int e = 0; e < 4; ++e) u[e] = fbits(v[e]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) u[e] = (j0 + e < n_cand) ? fbits(row[j0 + e]) : 0u;
    }
    int eq_cnt = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) eq_cnt += (j0 + e < n_cand && u[e] == tau) ? 1 : 0;
    int eq_total;
    int eq_rank = eq_seen + block_excl_scan(eq_cnt, tid, sh, eq_total);
    bool sel[4];
    int sel_cnt = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool valid = j0 + e < n_cand;
      const bool gt = valid && u[e] > tau;
      const bool eq = valid && u[e] == tau;
      sel[e] = gt || (eq && eq_rank < need_eq);
      eq_rank += eq ? 1 : 0;
      sel_cnt += sel[e] ? 1 : 0;
    }
    int sel_total;
    int opos = sel_seen + block_excl_scan(sel_cnt, tid, sh, sel_total);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (sel[e] && opos < p.topk) out[opos++] = (int32_t)(j0 + e);
    eq_seen += eq_total;
    sel_seen += sel_total;
  }
  for (int w = tid; w < p.window; w += SEL_THREADS) out[p.topk + w] = (int32_t)(n_cand + w);
  if (tid == 0) p.count[qid] = max_sel;
}

}  // namespace

size_t select_workspace_bytes(int, int, int64_t, int64_t) { return 0; }

hipError_t launch_select(const SelectParams& p, void*, size_t, hipStream_t stream) {
  if (p.B * p.n_q == 0) return hipSuccess;
  hipLaunchKernelGGL(select_kernel, dim3((unsigned)(p.B * p.n_q)), dim3(SEL_THREADS), 0, stream, p);
  return hipGetLastError();
}

}  // namespace hs2

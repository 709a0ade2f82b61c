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
// Design: one 512-thread workgroup per query row, four rows per CU.  Scores
// are >= 0, so their float32 bit patterns order like unsigned integers.
// Usually the row is read once: a 4096-score sample (128 blocks of 32) gives
// a threshold estimate that about 2 topk candidates reach; those are
// compacted into LDS in index order (up to 4096 of them) and an LDS radix
// select finds tau among them exactly.  The radix digits (10 bits, LDS
// histograms) start right below the bits common to the smallest and largest
// value searched, so they split the actual value range instead of the nearly
// constant exponent.  When the estimate keeps fewer than topk or more than
// 4096 candidates, an exact path reads the row again: a min/max pass, radix
// histogram passes, and a block-wide ordered compaction that stops as soon as
// topk candidates are out.
// Few long rows (at most 64 rows, at least 32768 candidates, the decode case)
// go to a multi-workgroup version of the same selection (below).
#include "hs2_device.hpp"
#include "hs2_internal.hpp"

namespace hs2 {
namespace {

constexpr int SEL_THREADS = 512;
constexpr int SEL_WAVES = SEL_THREADS / kWave;
constexpr int SEL_DIGIT = 10;
constexpr int SEL_BINS = 1 << SEL_DIGIT;

struct SelShared {
  int hist[SEL_BINS];
  int wave_tot[SEL_WAVES];
  int wave_tot2[2][SEL_WAVES];
  uint32_t wave_u[2 * SEL_WAVES];
  int pick_digit;
  int pick_above;
};

__device__ __forceinline__ uint32_t fbits(float x) { return __builtin_bit_cast(uint32_t, x); }

// v plus the value DPP control CTRL moves into this lane (0 where it moves
// none: lanes shifted in from outside the row, rows outside ROWMASK).
template <int CTRL, int ROWMASK = 0xf>
__device__ __forceinline__ int dpp_add(int v) {
  return v + __builtin_amdgcn_update_dpp(0, v, CTRL, ROWMASK, 0xf, false);
}

// Inclusive scan of v over the wave: Hillis-Steele steps inside each 16-lane
// row (row_shr 1, 2, 4, 8), then the row totals are carried across rows
// (row_bcast 15 into rows 1 and 3, row_bcast 31 into rows 2 and 3).
__device__ __forceinline__ int wave_incl_scan(int v, int /*lane*/) {
  v = dpp_add<0x111>(v);
  v = dpp_add<0x112>(v);
  v = dpp_add<0x114>(v);
  v = dpp_add<0x118>(v);
  v = dpp_add<0x142, 0xa>(v);
  v = dpp_add<0x143, 0xc>(v);
  return v;
}

// Exclusive block-wide scan with a single barrier.  The wave totals go to one
// of two slots, alternating per call (par, uniform over the block): a slot is
// rewritten two scans later, after every thread has passed the barrier of
// the scan in between and so has finished reading it.
__device__ __forceinline__ int block_excl_scan1(int v, int tid, SelShared& sh, int& par, int& total) {
  const int lane = tid & 63, wave = tid >> 6;
  const int inc = wave_incl_scan(v, lane);
  int* wt = sh.wave_tot2[par];
  if (lane == 63) wt[wave] = inc;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < SEL_WAVES; ++w) {
    const int t = wt[w];
    before += (w < wave) ? t : 0;
    total += t;
  }
  par ^= 1;
  return before + inc - v;
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

template <int NT>
__device__ __forceinline__ int block_excl_scan_n(int v, int tid, SelShared& sh, int& total) {
  const int lane = tid & 63, wave = tid >> 6;
  const int inc = wave_incl_scan(v, lane);
  if (lane == 63) sh.wave_tot[wave] = inc;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < NT / kWave; ++w) {
    const int t = sh.wave_tot[w];
    before += (w < wave) ? t : 0;
    total += t;
  }
  __syncthreads();
  return before + inc - v;
}

// Digit pick of one radix pass.  sh.hist holds the counts of nbins digits;
// thread t owns the SEL_BINS / SEL_THREADS digits below nbins - per * t, so
// the block scan runs from the top digit down.  The digit that holds the
// krem-th largest value goes to sh.pick_digit, the count above it to
// sh.pick_above (visible to every thread on return).
__device__ __forceinline__ void pick_digit(SelShared& sh, int nbins, int krem, int& par) {
  constexpr int PERB = SEL_BINS / SEL_THREADS;
  const int tid = threadIdx.x;
  int c[PERB];
  int mine = 0;
#pragma unroll
  for (int i = 0; i < PERB; ++i) {
    const int d = nbins - 1 - PERB * tid - i;
    c[i] = d >= 0 ? sh.hist[d] : 0;
    mine += c[i];
  }
  int total;
  int before = block_excl_scan1(mine, tid, sh, par, total);
#pragma unroll
  for (int i = 0; i < PERB; ++i) {
    const int d = nbins - 1 - PERB * tid - i;
    if (d >= 0 && before < krem && krem <= before + c[i]) {
      sh.pick_digit = d;
      sh.pick_above = before;
    }
    before += c[i];
  }
  __syncthreads();
}

// ---- sampled single-read path (the common case) ----------------------------
// Rows up to SEL_CAP candidates, and rows whose candidates at or above a
// threshold estimated from a sample of the row number between topk and SEL_CAP,
// are selected from one read of the row: the candidates at or above the
// estimate are compacted into LDS in index order, and tau is found there.
// Anything else (a sample that misleads, e.g. many equal scores) falls back to
// the exact multi-pass radix below, so the result never depends on the sample.
constexpr int SEL_CAP = 4096;      // candidates kept in LDS (32 KB: four rows share a CU)
constexpr int SEL_SAMPLE = 4096;   // sampled scores of a long row (128 blocks of 32)
constexpr int SEL_SPT = SEL_SAMPLE / SEL_THREADS;  // sampled scores per thread
static_assert(SEL_SAMPLE % (4 * SEL_THREADS) == 0 && SEL_CAP >= 32, "whole float4s per thread");

// Block-wide minimum and maximum of the per-thread lo and hi (returned to
// every thread); ends with a barrier, which also orders the LDS writes made
// before the call.
__device__ __forceinline__ void block_min_max(uint32_t& lo, uint32_t& hi, SelShared& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    hi = max(hi, (uint32_t)__shfl_xor((int)hi, o, kWave));
    lo = min(lo, (uint32_t)__shfl_xor((int)lo, o, kWave));
  }
  if (lane == 0) {
    sh.wave_u[wave] = hi;
    sh.wave_u[SEL_WAVES + wave] = lo;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < SEL_WAVES; ++w) {
    hi = max(hi, sh.wave_u[w]);
    lo = min(lo, sh.wave_u[SEL_WAVES + w]);
  }
}

// The k-th largest of the n bit patterns v[0..n-1] in LDS (k >= 1, n >= k),
// all of them in [lo, hi]: returns tau and how many of the values equal to
// tau rank inside the top k.  The bits above the highest bit where lo and hi
// differ are common to every value, so the 10-bit digits start right below
// them and split the actual range (few values share a histogram bin, which
// keeps the LDS atomics apart).  After max_pass digits the search stops:
// tau then has its lower bits 0, a lower bound of the k-th largest that only
// the values sharing all of its higher bits pass.
// Digits that resolve any 32-bit range (4 x 10 bits >= 32): the search is exact.
constexpr int kRadixExact = (32 + SEL_DIGIT - 1) / SEL_DIGIT;

__device__ void lds_radix_select(const uint32_t* v, int n, int k, uint32_t lo, uint32_t hi, int max_pass,
                                 SelShared& sh, int& par, uint32_t& tau, int& need_eq) {
  const int tid = threadIdx.x;
  int krem = k;
  if (lo == hi) {  // every value equal
    tau = lo;
    need_eq = krem;
    return;
  }
  int shift = 32 - __builtin_clz(lo ^ hi);
  uint64_t prefix = (uint64_t)hi >> shift << shift;
  for (int pass = 0; shift > 0 && pass < max_pass; ++pass) {
    const int w = min(SEL_DIGIT, shift);
    shift -= w;
    const int nbins = 1 << w;
    // 64-bit shifts: shift + w may be 32
    const uint64_t want = prefix >> (shift + w);
    for (int b = tid; b < nbins; b += SEL_THREADS) sh.hist[b] = 0;
    __syncthreads();
    for (int j = tid; j < n; j += SEL_THREADS) {
      const uint64_t u = v[j];
      if ((u >> (shift + w)) == want) atomicAdd(&sh.hist[(u >> shift) & (nbins - 1)], 1);
    }
    __syncthreads();
    pick_digit(sh, nbins, krem, par);
    prefix |= (uint64_t)sh.pick_digit << shift;
    krem -= sh.pick_above;
  }
  tau = (uint32_t)prefix;
  need_eq = krem;
}

__global__ __launch_bounds__(SEL_THREADS) __attribute__((amdgpu_waves_per_eu(8))) void select_kernel(const SelectParams p) {
  __shared__ SelShared sh;
  __shared__ uint32_t cval[SEL_CAP];
  __shared__ int32_t cidx[SEL_CAP];
  const int tid = threadIdx.x;
  const int qid = xcd_remap(blockIdx.x, gridDim.x);
  const int i = qid % p.n_q;
  const int64_t pos = p.q_pos0 + i;
  const int64_t n = pos + 1;
  const int max_sel = p.window + p.topk;
  int32_t* out = p.idx + (int64_t)qid * max_sel;
  const float* row = p.scores + (int64_t)qid * p.ld_scores;
  const int64_t n_cand = n > p.window ? n - p.window : 0;
  int par = 0;  // slot of the next single-barrier scan

  if (n_cand <= p.topk) {  // every key 0..p is selected
    for (int j = tid; j < max_sel; j += SEL_THREADS) out[j] = j < n ? j : -1;
    if (tid == 0) p.count[qid] = (int32_t)n;
    return;
  }

  // ---- sampled path: threshold estimate (0 = keep everything for short rows)
  uint32_t u_est = 0u;
  if (n_cand > SEL_CAP) {
    // 128 evenly spaced blocks of 32 consecutive scores, each one 128-byte
    // line: about 3 % of the row's bytes (single strided values would touch
    // up to every line of the row)
    uint32_t smin = 0xFFFFFFFFu, smax = 0u;
#pragma unroll
    for (int h = 0; h < SEL_SPT / 4; ++h) {
      const int i = tid + h * SEL_THREADS;
      const int64_t blk = i >> 3;
      const int64_t start = (blk * (n_cand - 32) / (SEL_SAMPLE / 32 - 1)) & ~(int64_t)31;
      const f32x4 v = *(const f32x4*)(row + start + 4 * (i & 7));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t u = fbits(v[e]);
        cval[4 * i + e] = u;
        smin = min(smin, u);
        smax = max(smax, u);
      }
    }
    block_min_max(smin, smax, sh);
    // aim at about 2 topk candidates at or above the estimate (less for a
    // topk above SEL_CAP / 3, to stay inside the LDS); two digits (20 bits
    // below the sample's common prefix) are precise enough
    const int64_t aim = min<int64_t>(2 * (int64_t)p.topk, ((int64_t)p.topk + SEL_CAP) / 2);
    const int r = (int)min<int64_t>(SEL_SAMPLE, max<int64_t>(1, (aim * SEL_SAMPLE + n_cand - 1) / n_cand));
    int unused;
    lds_radix_select(cval, SEL_SAMPLE, r, smin, smax, 2, sh, par, u_est, unused);
  }
  // one read of the row: candidates >= u_est into LDS, in index order.  A
  // round covers 4096 candidates: wave wv takes PIECE consecutive ones, its
  // kept positions come from ballots and mbcnt, and one barrier orders the
  // waves.  The loads of the next round are issued before the barrier.  The
  // smallest and largest kept pattern bound the exact search below.
  constexpr int PER = 8;
  constexpr int ROUND = PER * SEL_THREADS;  // candidates per round
  constexpr int PIECE = PER * kWave;        // consecutive candidates of one wave per round
  const int lane = tid & 63, wv = tid >> 6;
  // load q of lane l is the float4 at 256 q + 4 l of the wave's piece
  auto load16 = [&](int64_t base, uint32_t (&u)[PER]) {
#pragma unroll
    for (int q = 0; q < PER / 4; ++q) {
      const int64_t j = base + PIECE * wv + 256 * q + 4 * lane;
      if (j + 3 < n_cand) {
        const f32x4 v = *(const f32x4*)(row + j);
#pragma unroll
        for (int e = 0; e < 4; ++e) u[4 * q + e] = fbits(v[e]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) u[4 * q + e] = (j + e < n_cand) ? fbits(row[j + e]) : 0u;
      }
    }
  };
  int kept = 0;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  uint32_t ucur[PER], unext[PER];
  load16(0, ucur);
  for (int64_t base = 0; base < n_cand; base += ROUND) {
    if (base + ROUND < n_cand) load16(base + ROUND, unext);
    uint64_t bal[PER];
    int wtot = 0;
#pragma unroll
    for (int q = 0; q < PER / 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t j = base + PIECE * wv + 256 * q + 4 * lane + e;
        const bool keep = j < n_cand && ucur[4 * q + e] >= u_est;
        bal[4 * q + e] = __ballot(keep);
        wtot += __popcll(bal[4 * q + e]);
        kmin = min(kmin, keep ? ucur[4 * q + e] : 0xFFFFFFFFu);
        kmax = max(kmax, keep ? ucur[4 * q + e] : 0u);
      }
    int* wt = sh.wave_tot2[par];
    if (lane == 0) wt[wv] = wtot;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < SEL_WAVES; ++w) {
      const int t = wt[w];
      before += (w < wv) ? t : 0;
      tot += t;
    }
    par ^= 1;
    int pos = kept + before;
#pragma unroll
    for (int q = 0; q < PER / 4; ++q) {
      int p = pos;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        p += __builtin_amdgcn_mbcnt_hi((uint32_t)(bal[4 * q + e] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal[4 * q + e], 0));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if ((bal[4 * q + e] >> lane) & 1) {
          if (p < SEL_CAP) {
            cval[p] = ucur[4 * q + e];
            cidx[p] = (int32_t)(base + PIECE * wv + 256 * q + 4 * lane + e);
          }
          ++p;
        }
        pos += __popcll(bal[4 * q + e]);
      }
    }
    kept += tot;
#pragma unroll
    for (int e = 0; e < PER; ++e) ucur[e] = unext[e];
  }
  block_min_max(kmin, kmax, sh);
  if (kept >= p.topk && kept <= SEL_CAP) {
    // every pick is at or above u_est (at least topk candidates are), so the
    // exact tau of the row is the topk-th largest of the kept ones.  The pick
    // code below needs tau exact: the search runs until every bit below the
    // common prefix is resolved (a 31-bit range, e.g. scores on both sides of
    // 2.0 when they are summed over heads, takes 4 digits of 10 bits).
    uint32_t tau;
    int need_eq;
    lds_radix_select(cval, kept, p.topk, kmin, kmax, kRadixExact, sh, par, tau, need_eq);
    // a pick's output slot is the number of picks before it: the values above
    // tau before it plus the first need_eq ties.  One scan of the packed
    // counts (above << 16 | ties) per 4 * SEL_THREADS kept values.
    int gt_seen = 0, eq_seen = 0;
    for (int base = 0; base < kept; base += 4 * SEL_THREADS) {
      const int j0 = base + 4 * tid;
      uint32_t u[4];
      int ngt = 0, neq = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        u[e] = j0 + e < kept ? cval[j0 + e] : 0u;
        ngt += (j0 + e < kept && u[e] > tau) ? 1 : 0;
        neq += (j0 + e < kept && u[e] == tau) ? 1 : 0;
      }
      int tot;
      const int pre = block_excl_scan1((ngt << 16) | neq, tid, sh, par, tot);
      int gt_b = gt_seen + (pre >> 16), eq_b = eq_seen + (pre & 0xffff);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (j0 + e >= kept) continue;
        if (u[e] > tau) {
          const int opos = gt_b + min(eq_b, need_eq);
          if (opos < p.topk) out[opos] = cidx[j0 + e];
          ++gt_b;
        } else if (u[e] == tau) {
          if (eq_b < need_eq && gt_b + eq_b < p.topk) out[gt_b + eq_b] = cidx[j0 + e];
          ++eq_b;
        }
      }
      gt_seen += tot >> 16;
      eq_seen += tot & 0xffff;
    }
    for (int w = tid; w < p.window; w += SEL_THREADS) out[p.topk + w] = (int32_t)(n_cand + w);
    if (tid == 0) p.count[qid] = max_sel;
    return;
  }
  // the estimate was off (too few or too many kept): exact multi-pass radix

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
      pick_digit(sh, nbins, krem, par);
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

// ---------------------------------------------------------------------------
// Few long rows (decode): the same selection, spread over many workgroups per
// row.  The radix digits are fixed (bits 30-20, 19-9, 8-0 of the non-negative
// float32 pattern); each pass is one launch that histograms its segment of
// the row (LDS, then integer atomics into the row's global histogram, so the
// counts do not depend on the order).  Every workgroup of a later launch
// derives the digits picked so far from those histograms itself.  Then one
// launch counts, per segment, the candidates above tau and equal to tau, and
// the last one writes each segment's picks at their ascending positions.
constexpr int MB_THREADS = 256;
constexpr int MB_PER_THREAD = 16;
constexpr int MB_SEG = MB_THREADS * MB_PER_THREAD;  // candidates per workgroup
constexpr int MB_MAX_ROWS = 64;
constexpr int MB_MIN_CAND = 32768;
constexpr int MB_BINS = 2048;

struct MbWs {
  int* hist;     // [rows][3][MB_BINS]
  int* bcount;   // [rows][nblk][2]: candidates above tau, equal to tau
  int nblk;
};

__device__ __forceinline__ int mb_shift(int pass) { return pass == 0 ? 20 : (pass == 1 ? 9 : 0); }
__device__ __forceinline__ int mb_width(int pass) { return pass == 2 ? 9 : 11; }

struct MbShared {
  int part[MB_THREADS];
  int digit, above;
  int cnt[2 * MB_THREADS / kWave];
  int lh[MB_BINS];
};

// Digits of passes 0..npass-1 from the row's histograms: returns the common
// prefix (bits above the next digit) and how many picks remain inside it.
__device__ void mb_prefix(const int* hist_row, int npass, int topk, MbShared& sh, uint32_t& prefix, int& krem) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  prefix = 0u;
  krem = topk;
  for (int pass = 0; pass < npass; ++pass) {
    const int nb = 1 << mb_width(pass);
    const int per = nb / MB_THREADS;             // 8 (11-bit digits) or 2 (9-bit)
    const int* h = hist_row + pass * MB_BINS;
    // thread t owns digits nb-1-per*t down to nb-per*(t+1): the scan runs from
    // the top digit down
    int c = 0;
    for (int i = 0; i < per; ++i) c += h[nb - 1 - per * tid - i];
    const int inc = wave_incl_scan(c, lane);
    if (lane == 63) sh.cnt[wave] = inc;
    __syncthreads();
    int before = inc - c;
    for (int w = 0; w < wave; ++w) before += sh.cnt[w];
    if (before < krem && krem <= before + c) {   // exactly one thread: the total is >= krem
      int cum = before, d = nb - 1 - per * tid;
      for (int i = 0; i < per - 1; ++i, --d) {
        const int hv = h[d];
        if (cum + hv >= krem) break;
        cum += hv;
      }
      sh.digit = d;
      sh.above = cum;
    }
    __syncthreads();
    prefix |= (uint32_t)sh.digit << mb_shift(pass);
    krem -= sh.above;
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void mb_zero_kernel(int* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0;
}

template <int PASS>
__global__ __launch_bounds__(MB_THREADS) void mb_hist_kernel(const SelectParams p, const MbWs ws) {
  __shared__ MbShared sh;
  const int tid = threadIdx.x, row = blockIdx.y;
  const int64_t n_cand = p.q_pos0 + row % p.n_q + 1 - p.window;
  const int64_t s0 = (int64_t)blockIdx.x * MB_SEG;
  if (n_cand <= p.topk || s0 >= n_cand) return;
  int* hist_row = ws.hist + (int64_t)row * 3 * MB_BINS;
  uint32_t prefix;
  int krem;
  mb_prefix(hist_row, PASS, p.topk, sh, prefix, krem);
  for (int b = tid; b < MB_BINS; b += MB_THREADS) sh.lh[b] = 0;
  __syncthreads();
  const int sh_lo = mb_shift(PASS), w = mb_width(PASS);
  const uint32_t want = PASS == 0 ? 0u : prefix >> (sh_lo + w);
  const float* rowp = p.scores + (int64_t)row * p.ld_scores;
#pragma unroll
  for (int r = 0; r < MB_PER_THREAD / 4; ++r) {
    const int64_t j = s0 + 1024 * r + 4 * tid;
    uint32_t u[4];
    if (j + 3 < n_cand) {
      const f32x4 v = *(const f32x4*)(rowp + j);
#pragma unroll
      for (int e = 0; e < 4; ++e) u[e] = fbits(v[e]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) u[e] = (j + e < n_cand) ? fbits(rowp[j + e]) : 0xFFFFFFFFu;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (u[e] != 0xFFFFFFFFu && (u[e] >> (sh_lo + w)) == want) atomicAdd(&sh.lh[(u[e] >> sh_lo) & ((1 << w) - 1)], 1);
  }
  __syncthreads();
  int* gh = hist_row + PASS * MB_BINS;
  for (int b = tid; b < (1 << w); b += MB_THREADS)
    if (sh.lh[b]) atomicAdd(&gh[b], sh.lh[b]);
}

// Candidates above tau and equal to tau in each segment.
__global__ __launch_bounds__(MB_THREADS) void mb_count_kernel(const SelectParams p, const MbWs ws) {
  __shared__ MbShared sh;
  const int tid = threadIdx.x, row = blockIdx.y;
  const int64_t n_cand = p.q_pos0 + row % p.n_q + 1 - p.window;
  const int64_t s0 = (int64_t)blockIdx.x * MB_SEG;
  if (n_cand <= p.topk || s0 >= n_cand) return;
  uint32_t tau;
  int need_eq;
  mb_prefix(ws.hist + (int64_t)row * 3 * MB_BINS, 3, p.topk, sh, tau, need_eq);
  const float* rowp = p.scores + (int64_t)row * p.ld_scores;
  int above = 0, eq = 0;
#pragma unroll
  for (int r = 0; r < MB_PER_THREAD / 4; ++r) {
    const int64_t j = s0 + 1024 * r + 4 * tid;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (j + e < n_cand) {
        const uint32_t u = fbits(rowp[j + e]);
        above += u > tau;
        eq += u == tau;
      }
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    above += __shfl_xor(above, o, kWave);
    eq += __shfl_xor(eq, o, kWave);
  }
  if ((tid & 63) == 0) {
    sh.cnt[2 * (tid >> 6)] = above;
    sh.cnt[2 * (tid >> 6) + 1] = eq;
  }
  __syncthreads();
  if (tid == 0) {
    int a = 0, q = 0;
    for (int wv = 0; wv < MB_THREADS / kWave; ++wv) {
      a += sh.cnt[2 * wv];
      q += sh.cnt[2 * wv + 1];
    }
    int* bc = ws.bcount + ((int64_t)row * ws.nblk + blockIdx.x) * 2;
    bc[0] = a;
    bc[1] = q;
  }
}

// Each segment writes its picks at their ascending positions; segment 0 also
// writes the window, the count, and the rows that keep every key.
__global__ __launch_bounds__(MB_THREADS) void mb_write_kernel(const SelectParams p, const MbWs ws) {
  __shared__ MbShared sh;
  __shared__ SelShared ssh;
  const int tid = threadIdx.x, row = blockIdx.y;
  const int64_t pos = p.q_pos0 + row % p.n_q;
  const int64_t n = pos + 1;
  const int64_t n_cand = n - p.window;
  const int max_sel = p.window + p.topk;
  int32_t* out = p.idx + (int64_t)row * max_sel;
  const int64_t s0 = (int64_t)blockIdx.x * MB_SEG;
  if (n_cand <= p.topk) {
    if (blockIdx.x == 0) {
      for (int j = tid; j < max_sel; j += MB_THREADS) out[j] = j < n ? j : -1;
      if (tid == 0) p.count[row] = (int32_t)n;
    }
    return;
  }
  if (blockIdx.x == 0) {
    for (int w = tid; w < p.window; w += MB_THREADS) out[p.topk + w] = (int32_t)(n_cand + w);
    if (tid == 0) p.count[row] = max_sel;
  }
  if (s0 >= n_cand) return;
  uint32_t tau;
  int need_eq;
  mb_prefix(ws.hist + (int64_t)row * 3 * MB_BINS, 3, p.topk, sh, tau, need_eq);
  // picks and ties in the segments before this one
  int sel_before = 0, eq_before = 0;
  const int* bc = ws.bcount + (int64_t)row * ws.nblk * 2;
  for (int b = tid; b < (int)blockIdx.x; b += MB_THREADS) {
    sel_before += bc[2 * b];
    eq_before += bc[2 * b + 1];
  }
  int tot;
  (void)block_excl_scan_n<MB_THREADS>(sel_before, tid, ssh, tot);
  sel_before = tot;
  (void)block_excl_scan_n<MB_THREADS>(eq_before, tid, ssh, tot);
  eq_before = tot;
  // ties taken before this segment: the first need_eq ties in index order
  sel_before += min(eq_before, need_eq);
  const float* rowp = p.scores + (int64_t)row * p.ld_scores;
  int eq_seen = eq_before, sel_seen = sel_before;
#pragma unroll
  for (int r = 0; r < MB_PER_THREAD / 4; ++r) {
    const int64_t j0 = s0 + 1024 * r + 4 * tid;
    uint32_t u[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) u[e] = (j0 + e < n_cand) ? fbits(rowp[j0 + e]) : 0u;
    int eq_cnt = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) eq_cnt += (j0 + e < n_cand && u[e] == tau) ? 1 : 0;
    int eq_total;
    int eq_rank = eq_seen + block_excl_scan_n<MB_THREADS>(eq_cnt, tid, ssh, eq_total);
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
    int opos = sel_seen + block_excl_scan_n<MB_THREADS>(sel_cnt, tid, ssh, sel_total);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (sel[e] && opos < p.topk) out[opos++] = (int32_t)(j0 + e);
    eq_seen += eq_total;
    sel_seen += sel_total;
  }
}

bool select_multi_block(int B, int n_q, int64_t q_pos0, int window) {
  const int64_t max_cand = q_pos0 + n_q - window;
  return (int64_t)B * n_q <= MB_MAX_ROWS && max_cand >= MB_MIN_CAND;
}

size_t mb_layout(int rows, int64_t max_cand, char* base, MbWs* ws) {
  const int nblk = (int)((max_cand + MB_SEG - 1) / MB_SEG);
  const size_t hist_bytes = ((size_t)rows * 3 * MB_BINS * 4 + 255) & ~(size_t)255;
  const size_t cnt_bytes = ((size_t)rows * nblk * 2 * 4 + 255) & ~(size_t)255;
  if (ws) {
    ws->hist = (int*)base;
    ws->bcount = (int*)(base + hist_bytes);
    ws->nblk = nblk;
  }
  return hist_bytes + cnt_bytes;
}

// ---- block-level selection (the granularity token-level selection replaces) ----
// HySparse2 pages: agihunt.info summary, ablation paragraph (token-level against
// block-level selection at the same 1024-token budget, blocks of 64); 10100.com
// article, section on the first refinement.  For the query at position p the
// candidates C = [0, p-window] are cut into aligned blocks of `block` tokens
// (the last one may be partial); a block scores the sum of its candidates'
// scores as a float32 pairwise tree (adjacent pairs first); the topk / block
// best blocks are kept, ties to the lower block, and the window is added.
//
// Two kernels.  block_sum_kernel streams the score rows once: each lane sums
// its float4 ((x0 + x1) + (x2 + x3)) and the block / 4 lanes of a block
// combine by xor-shuffles 1, 2, 4, ..., which is exactly the pairwise tree.
// block_select_kernel (one workgroup per row) loads the row's block sums into
// LDS, finds the topk / block-th largest with the LDS radix select above and
// writes the token indices in ascending order.
constexpr int BK_THREADS = 256;
constexpr int BK_UNROLL = 8;
constexpr int BK_FLOATS = BK_THREADS * BK_UNROLL * 4;  // scores per block-sum workgroup

__device__ __forceinline__ int64_t bk_cand(const SelectParams& p, int64_t row) {
  return p.q_pos0 + row % p.n_q + 1 - p.window;  // |C| (may be <= 0)
}

template <int LPB>  // lanes per block = block / 4
__global__ __launch_bounds__(BK_THREADS) void block_sum_kernel(const SelectParams p, int64_t row0, int nchunk,
                                                               int nb_max, float* __restrict__ bsum) {
  constexpr int block = 4 * LPB;
  const int64_t row = row0 + blockIdx.x / nchunk;
  const int chunk = blockIdx.x % nchunk;
  const int64_t n_cand = bk_cand(p, row);
  if (n_cand <= p.topk) return;  // every key is selected: no sums needed
  const int64_t nb = (n_cand + block - 1) / block;
  const int64_t f0 = (int64_t)chunk * BK_FLOATS;
  if (f0 >= n_cand) return;
  const float* src = p.scores + row * p.ld_scores;
  const int tid = threadIdx.x;
  f32x4 x[BK_UNROLL];
  // f < n_cand <= ld_scores with f and ld_scores multiples of 4: the float4 is inside the row
#pragma unroll
  for (int it = 0; it < BK_UNROLL; ++it) {
    const int64_t f = f0 + 4 * (it * BK_THREADS + tid);
    x[it] = f < n_cand ? *(const f32x4*)(src + f) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int it = 0; it < BK_UNROLL; ++it) {
    const int64_t f = f0 + 4 * (it * BK_THREADS + tid);
    f32x4 v = x[it];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = f + e < n_cand ? v[e] : 0.f;  // scores past C (the window) count 0
    float t = (v[0] + v[1]) + (v[2] + v[3]);
#pragma unroll
    for (int m = 1; m < LPB; m <<= 1) t += shfl_xor(t, m);
    const int64_t b = f / block;
    if ((tid % LPB) == 0 && b < nb) bsum[(row - row0) * nb_max + b] = t;
  }
}

constexpr int BK_MAX_IDS = kMaxSelect / 4;  // selected blocks: topk / block with block >= 4

template <int CAP>
__global__ __launch_bounds__(SEL_THREADS) void block_select_kernel(const SelectParams p, int64_t row0, int block,
                                                                   int nb_max, const float* __restrict__ bsum) {
  __shared__ SelShared sh;
  __shared__ uint32_t bv[CAP];
  __shared__ int sel_ids[BK_MAX_IDS];
  const int64_t row = row0 + blockIdx.x;
  const int tid = threadIdx.x;
  const int max_sel = p.window + p.topk;
  const int64_t n = p.q_pos0 + row % p.n_q + 1;
  const int64_t n_cand = n - p.window;
  int32_t* out = p.idx + row * max_sel;
  if (n_cand <= p.topk) {
    for (int j = tid; j < max_sel; j += SEL_THREADS) out[j] = j < n ? j : -1;
    if (tid == 0) p.count[row] = (int32_t)n;
    return;
  }
  const int nb = (int)((n_cand + block - 1) / block);
  const int nsel = p.topk / block;
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
  const float* src = bsum + (row - row0) * nb_max;
  for (int b = tid; b < nb; b += SEL_THREADS) {
    const uint32_t u = fbits(src[b]);
    bv[b] = u;
    lo = min(lo, u);
    hi = max(hi, u);
  }
  block_min_max(lo, hi, sh);  // ends with a barrier: bv is complete
  int par = 0;
  uint32_t tau;
  int need_eq;
  lds_radix_select(bv, nb, nsel, lo, hi, kRadixExact, sh, par, tau, need_eq);
  // thread t owns the blocks [t*per, (t+1)*per): two ordered scans give the
  // equal-to-tau rank and then the output rank of each selected block
  const int per = (nb + SEL_THREADS - 1) / SEL_THREADS;
  const int b0 = min(nb, tid * per), b1 = min(nb, b0 + per);
  int my_eq = 0;
  for (int b = b0; b < b1; ++b) my_eq += bv[b] == tau;
  int total;
  int eq_before = block_excl_scan(my_eq, tid, sh, total);
  int my_sel = 0;
  for (int b = b0, e = eq_before; b < b1; ++b) {
    const uint32_t u = bv[b];
    if (u > tau || (u == tau && e++ < need_eq)) ++my_sel;
  }
  int rank = block_excl_scan(my_sel, tid, sh, total);
  for (int b = b0, e = eq_before; b < b1; ++b) {
    const uint32_t u = bv[b];
    if (u > tau || (u == tau && e++ < need_eq)) sel_ids[rank++] = b;
  }
  __syncthreads();
  const int64_t last = sel_ids[nsel - 1];
  const int nbt = (nsel - 1) * block + (int)min((int64_t)block, n_cand - last * block);
  for (int j = tid; j < max_sel; j += SEL_THREADS) {
    int32_t v;
    if (j < nbt) v = (int32_t)((int64_t)sel_ids[j / block] * block + j % block);
    else if (j < nbt + p.window) v = (int32_t)(n_cand + (j - nbt));
    else v = -1;
    out[j] = v;
  }
  if (tid == 0) p.count[row] = nbt + p.window;
}

}  // namespace

// Sized for the smallest window (1), which has the most candidates: the launch
// with the caller's window needs at most this much, or none.
size_t select_workspace_bytes(int B, int n_q, int64_t /*T*/, int64_t q_pos0) {
  if (!select_multi_block(B, n_q, q_pos0, 1)) return 0;
  return mb_layout(B * n_q, q_pos0 + n_q - 1, nullptr, nullptr);
}

hipError_t launch_select(const SelectParams& p, void* ws_ptr, size_t /*ws_bytes*/, hipStream_t stream) {
  if (p.B * p.n_q == 0) return hipSuccess;
  if (!select_multi_block(p.B, p.n_q, p.q_pos0, p.window)) {
    hipLaunchKernelGGL(select_kernel, dim3((unsigned)(p.B * p.n_q)), dim3(SEL_THREADS), 0, stream, p);
    return hipGetLastError();
  }
  const int rows = p.B * p.n_q;
  MbWs ws;
  mb_layout(rows, p.q_pos0 + p.n_q - p.window, (char*)ws_ptr, &ws);
  const int64_t nh = (int64_t)rows * 3 * MB_BINS;
  hipLaunchKernelGGL(mb_zero_kernel, dim3((unsigned)((nh + 255) / 256 < 1024 ? (nh + 255) / 256 : 1024)), dim3(256), 0,
                     stream, ws.hist, nh);
  const dim3 grid((unsigned)ws.nblk, (unsigned)rows);
  hipLaunchKernelGGL(mb_hist_kernel<0>, grid, dim3(MB_THREADS), 0, stream, p, ws);
  hipLaunchKernelGGL(mb_hist_kernel<1>, grid, dim3(MB_THREADS), 0, stream, p, ws);
  hipLaunchKernelGGL(mb_hist_kernel<2>, grid, dim3(MB_THREADS), 0, stream, p, ws);
  hipLaunchKernelGGL(mb_count_kernel, grid, dim3(MB_THREADS), 0, stream, p, ws);
  hipLaunchKernelGGL(mb_write_kernel, grid, dim3(MB_THREADS), 0, stream, p, ws);
  return hipGetLastError();
}

int64_t select_blocks_nb_max(int64_t q_pos0, int n_q, int window, int block) {
  const int64_t c = q_pos0 + n_q - window;  // candidates of the last row
  return c > 0 ? (c + block - 1) / block : 0;
}

size_t select_blocks_workspace_bytes(int B, int n_q, int64_t q_pos0, int window, int block) {
  return (((size_t)B * n_q * (size_t)select_blocks_nb_max(q_pos0, n_q, window, block) * 4) + 255) & ~(size_t)255;
}

hipError_t launch_select_blocks(const SelectParams& p, int block, void* ws_ptr, hipStream_t stream) {
  const int64_t rows = (int64_t)p.B * p.n_q;
  if (rows == 0) return hipSuccess;
  const int nb_max = (int)select_blocks_nb_max(p.q_pos0, p.n_q, p.window, block);
  const int nchunk = nb_max > 0 ? (int)(((int64_t)nb_max * block + BK_FLOATS - 1) / BK_FLOATS) : 0;
  float* bsum = (float*)ws_ptr;
  // rows per launch: keep every grid under 2^31 work-items
  const int64_t step = (int64_t)(1u << 31) / ((int64_t)BK_THREADS * (nchunk > 0 ? nchunk : 1) + SEL_THREADS);
  for (int64_t r0 = 0; r0 < rows; r0 += step) {
    const int64_t nr = rows - r0 < step ? rows - r0 : step;
    if (nchunk > 0) {
      const dim3 g((unsigned)(nr * nchunk));
      float* bs = bsum + r0 * nb_max;
      switch (block) {
        case 4: hipLaunchKernelGGL(block_sum_kernel<1>, g, dim3(BK_THREADS), 0, stream, p, r0, nchunk, nb_max, bs); break;
        case 8: hipLaunchKernelGGL(block_sum_kernel<2>, g, dim3(BK_THREADS), 0, stream, p, r0, nchunk, nb_max, bs); break;
        case 16: hipLaunchKernelGGL(block_sum_kernel<4>, g, dim3(BK_THREADS), 0, stream, p, r0, nchunk, nb_max, bs); break;
        case 32: hipLaunchKernelGGL(block_sum_kernel<8>, g, dim3(BK_THREADS), 0, stream, p, r0, nchunk, nb_max, bs); break;
        case 64: hipLaunchKernelGGL(block_sum_kernel<16>, g, dim3(BK_THREADS), 0, stream, p, r0, nchunk, nb_max, bs); break;
        case 128: hipLaunchKernelGGL(block_sum_kernel<32>, g, dim3(BK_THREADS), 0, stream, p, r0, nchunk, nb_max, bs); break;
        default: hipLaunchKernelGGL(block_sum_kernel<64>, g, dim3(BK_THREADS), 0, stream, p, r0, nchunk, nb_max, bs); break;
      }
    }
    const float* bs = bsum + r0 * nb_max;
    if (nb_max <= 4096)
      hipLaunchKernelGGL(block_select_kernel<4096>, dim3((unsigned)nr), dim3(SEL_THREADS), 0, stream, p, r0, block,
                         nb_max, bs);
    else
      hipLaunchKernelGGL(block_select_kernel<kMaxBlocks>, dim3((unsigned)nr), dim3(SEL_THREADS), 0, stream, p,
                         r0, block, nb_max, bs);
  }
  return hipGetLastError();
}

}  // namespace hs2

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

// Threshold estimate for a row of more than SEL_CAP candidates: the bit
// pattern that about `aim` candidates reach, from 128 evenly spaced blocks of
// 32 consecutive scores (each one 128-byte line: about 3 % of a 114k row;
// single strided values would touch up to every line of the row).  Two
// digits (20 bits below the sample's common prefix) are precise enough.
// cval is LDS scratch of SEL_SAMPLE entries.
__device__ __forceinline__ uint32_t sample_estimate(const float* row, int64_t n_cand, int64_t aim, uint32_t* cval,
                                                    SelShared& sh, int& par) {
  const int tid = threadIdx.x;
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
  const int r = (int)min<int64_t>(SEL_SAMPLE, max<int64_t>(1, (aim * SEL_SAMPLE + n_cand - 1) / n_cand));
  uint32_t u_est;
  int unused;
  lds_radix_select(cval, SEL_SAMPLE, r, smin, smax, 2, sh, par, u_est, unused);
  return u_est;
}

// The topk picks among kept candidates held in LDS in index order
// (cval/cidx[0..kept), topk <= kept, every pick among them, patterns in
// [kmin, kmax]) -> out[0..topk), ascending.  tau is found exactly: the
// search runs until every bit below the common prefix is resolved (a 31-bit
// range, e.g. scores on both sides of 2.0 when they are summed over heads,
// takes 4 digits of 10 bits).  A pick's output slot is the number of picks
// before it: the values above tau before it plus the first need_eq ties; one
// scan of the packed counts (above << 16 | ties) per 4 * SEL_THREADS values.
__device__ __forceinline__ void pick_from_lds(const uint32_t* cval, const int32_t* cidx, int kept, uint32_t kmin,
                                              uint32_t kmax, int topk, int32_t* out, SelShared& sh, int& par) {
  const int tid = threadIdx.x;
  uint32_t tau;
  int need_eq;
  lds_radix_select(cval, kept, topk, kmin, kmax, kRadixExact, sh, par, tau, need_eq);
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
        if (opos < topk) out[opos] = cidx[j0 + e];
        ++gt_b;
      } else if (u[e] == tau) {
        if (eq_b < need_eq && gt_b + eq_b < topk) out[gt_b + eq_b] = cidx[j0 + e];
        ++eq_b;
      }
    }
    gt_seen += tot >> 16;
    eq_seen += tot & 0xffff;
  }
}

// The exact multi-pass selection over a whole row of n_cand > topk
// candidates -> out[0..topk), ascending: a min/max pass, radix histogram
// passes below the common prefix, then a block-wide ordered compaction that
// stops as soon as topk candidates are out.
__device__ void exact_row(const float* row, int64_t n_cand, int topk, int32_t* out, SelShared& sh, int& par) {
  const int tid = threadIdx.x;
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
  block_min_max(mn, mx, sh);

  // ---- radix passes below the common prefix
  uint32_t tau;
  int need_eq;  // how many candidates equal to tau are taken (in index order)
  if (mx == mn) {
    tau = mx;
    need_eq = topk;
  } else {
    const int hb = 31 - __builtin_clz(mx ^ mn);
    int shift = hb + 1;
    uint64_t prefix = (uint64_t)mx >> shift << shift;  // common high bits
    int krem = topk;
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
  for (int64_t base = 0; base < n_cand && sel_seen < topk; base += 4 * SEL_THREADS) {
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
      if (sel[e] && opos < topk) out[opos++] = (int32_t)(j0 + e);
    eq_seen += eq_total;
    sel_seen += sel_total;
  }
}

// One read of candidates [c0, c0 + 8 * SEL_THREADS) of a row (n_cand of
// them): wave wv takes the 512 consecutive ones from c0 + 512 wv, lane l the
// float4s at 256 q + 4 l of that piece.  Entries at or past n_cand hold
// whatever the row has there: every caller tests round_index < n_cand before
// it uses an entry.
constexpr int SEL_PER = 8;
constexpr int SEL_ROUND = SEL_PER * SEL_THREADS;  // candidates per round
constexpr int SEL_PIECE = SEL_PER * kWave;        // consecutive candidates of one wave per round
__device__ __forceinline__ void load_round(const float* row, int64_t n_cand, int64_t c0, uint32_t (&u)[SEL_PER]) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int q = 0; q < SEL_PER / 4; ++q) {
    const int64_t j = c0 + SEL_PIECE * wv + 256 * q + 4 * lane;
    // One float4 load on every path and no use of the data here, so that the
    // compiler counts the loads in flight and waits only where the entries
    // are used (a load under a condition, or a select on the loaded value,
    // made it wait right after the loads, which undid the prefetch of the
    // next round).  j is a multiple of 4 and a row holds a multiple of 4
    // scores, more than n_cand, so the float4 at j < n_cand lies inside the
    // row; lanes past the candidates read the row's first float4.
    const f32x4 v = *(const f32x4*)(row + (j < n_cand ? j : 0));
#pragma unroll
    for (int e = 0; e < 4; ++e) u[4 * q + e] = fbits(v[e]);
  }
}
__device__ __forceinline__ int64_t round_index(int64_t c0, int q, int e) {
  return c0 + SEL_PIECE * (threadIdx.x >> 6) + 256 * q + 4 * (threadIdx.x & 63) + e;
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
  // aiming at about 2 topk candidates (less for a topk above SEL_CAP / 3, to
  // stay inside the LDS)
  uint32_t u_est = 0u;
  if (n_cand > SEL_CAP)
    u_est = sample_estimate(row, n_cand, min<int64_t>(2 * (int64_t)p.topk, ((int64_t)p.topk + SEL_CAP) / 2), cval,
                            sh, par);
  // one read of the row: candidates >= u_est into LDS, in index order.  A
  // round covers 4096 candidates: each wave takes SEL_PIECE consecutive ones,
  // its kept positions come from ballots and mbcnt, and one barrier orders the
  // waves.  The loads of the next round are issued before the barrier.  The
  // smallest and largest kept pattern bound the exact search below.
  const int lane = tid & 63, wv = tid >> 6;
  int kept = 0;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  uint32_t ucur[SEL_PER], unext[SEL_PER];
  load_round(row, n_cand, 0, ucur);
  for (int64_t base = 0; base < n_cand; base += SEL_ROUND) {
    load_round(row, n_cand, base + SEL_ROUND, unext);   // past the row: its first float4s, never used
    __builtin_amdgcn_sched_barrier(0);                  // the next round's loads go out first
    uint64_t bal[SEL_PER];
    int wtot = 0;
#pragma unroll
    for (int q = 0; q < SEL_PER / 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool keep = round_index(base, q, e) < n_cand && ucur[4 * q + e] >= u_est;
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
    for (int q = 0; q < SEL_PER / 4; ++q) {
      int p = pos;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        p += __builtin_amdgcn_mbcnt_hi((uint32_t)(bal[4 * q + e] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal[4 * q + e], 0));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if ((bal[4 * q + e] >> lane) & 1) {
          if (p < SEL_CAP) {
            cval[p] = ucur[4 * q + e];
            cidx[p] = (int32_t)round_index(base, q, e);
          }
          ++p;
        }
        pos += __popcll(bal[4 * q + e]);
      }
    }
    kept += tot;
#pragma unroll
    for (int e = 0; e < SEL_PER; ++e) ucur[e] = unext[e];
  }
  block_min_max(kmin, kmax, sh);
  // every pick is at or above u_est when at least topk candidates are, so the
  // exact tau of the row is the topk-th largest of the kept ones; otherwise
  // (the estimate was off: too few or too many kept) the exact multi-pass radix
  if (kept >= p.topk && kept <= SEL_CAP)
    pick_from_lds(cval, cidx, kept, kmin, kmax, p.topk, out, sh, par);
  else
    exact_row(row, n_cand, p.topk, out, sh, par);
  for (int w = tid; w < p.window; w += SEL_THREADS) out[p.topk + w] = (int32_t)(n_cand + w);
  if (tid == 0) p.count[qid] = max_sel;
}

// ---------------------------------------------------------------------------
// Few long rows (decode: at most 64 rows of at least FR_MIN_CAND candidates):
// the same selection with the row's one read spread over many workgroups.
//   fr_compact_kernel: grid (segments of 4096 candidates, rows).  Every
//     workgroup of a row derives the same threshold estimate from the same
//     sample (no launch and no wait for it), then compacts the candidates of
//     its segment at or above it, in index order, into the segment's slot of
//     the workspace (at most FR_SCAP of them) and writes how many there are.
//   fr_final_kernel: one workgroup per row.  A scan of the segment counts
//     places each segment's candidates; they are gathered into LDS in index
//     order (a segment that kept more than its slot holds is read again from
//     the row), and the LDS selection of the single-read path picks tau and
//     the output.  When the estimate kept fewer than topk or more than
//     FR_KCAP candidates, the exact multi-pass selection reads the row instead.
// Every count has its own slot and every position comes from a scan, so the
// result does not depend on timing; nothing needs clearing between calls.
constexpr int FR_SEG = SEL_ROUND;   // candidates per segment workgroup (one round)
constexpr int FR_SCAP = 512;        // kept candidates stored per segment
constexpr int FR_KCAP = 8192;       // kept candidates of a row gathered into LDS (64 KB)
constexpr int FR_MAX_ROWS = 64;
constexpr int FR_MIN_CAND = 24576;

struct FrWs {
  uint32_t* u_est;   // [rows]: the threshold estimate of each row
  int* count;        // [rows][nseg]: candidates at or above it in each segment
  uint2* kept;       // [rows][nseg][FR_SCAP]: (pattern, index) of the first FR_SCAP of them
  int nseg;
};

// about 3 topk candidates at or above the estimate: a sample of 4096 then
// misses below topk or above FR_KCAP rarely even on rows of 2^20 candidates
__device__ __forceinline__ int64_t fr_aim(int topk) {
  return min<int64_t>(3 * (int64_t)topk, ((int64_t)topk + FR_KCAP) / 2);
}

__global__ __launch_bounds__(SEL_THREADS) void fr_compact_kernel(const SelectParams p, const FrWs ws) {
  __shared__ SelShared sh;
  __shared__ uint32_t cval[SEL_SAMPLE];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int row = blockIdx.y, seg = blockIdx.x;
  const int64_t n_cand = p.q_pos0 + row % p.n_q + 1 - p.window;
  const int64_t c0 = (int64_t)seg * FR_SEG;
  if (n_cand <= p.topk || c0 >= n_cand) return;
  const float* rowp = p.scores + (int64_t)row * p.ld_scores;
  uint32_t u[SEL_PER];
  load_round(rowp, n_cand, c0, u);   // in flight during the estimate
  int par = 0;
  const uint32_t u_est = sample_estimate(rowp, n_cand, fr_aim(p.topk), cval, sh, par);
  uint64_t bal[SEL_PER];
  int wtot = 0;
#pragma unroll
  for (int q = 0; q < SEL_PER / 4; ++q)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool keep = round_index(c0, q, e) < n_cand && u[4 * q + e] >= u_est;
      bal[4 * q + e] = __ballot(keep);
      wtot += __popcll(bal[4 * q + e]);
    }
  int* wt = sh.wave_tot2[par];
  if (lane == 0) wt[wv] = wtot;
  __syncthreads();
  int pos = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < SEL_WAVES; ++w) {
    const int t = wt[w];
    pos += (w < wv) ? t : 0;
    tot += t;
  }
  const int64_t slot = (int64_t)row * ws.nseg + seg;
  uint2* dst = ws.kept + slot * FR_SCAP;
#pragma unroll
  for (int q = 0; q < SEL_PER / 4; ++q) {
    int pp = pos;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      pp += __builtin_amdgcn_mbcnt_hi((uint32_t)(bal[4 * q + e] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal[4 * q + e], 0));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if ((bal[4 * q + e] >> lane) & 1) {
        if (pp < FR_SCAP) dst[pp] = make_uint2(u[4 * q + e], (uint32_t)round_index(c0, q, e));
        ++pp;
      }
      pos += __popcll(bal[4 * q + e]);
    }
  }
  if (tid == 0) {
    ws.count[slot] = tot;
    if (seg == 0) ws.u_est[row] = u_est;
  }
}

__global__ __launch_bounds__(SEL_THREADS) void fr_final_kernel(const SelectParams p, const FrWs ws) {
  __shared__ SelShared sh;
  __shared__ uint32_t cval[FR_KCAP];
  __shared__ int32_t cidx[FR_KCAP];
  __shared__ int seg_cnt[SEL_THREADS], seg_pos[SEL_THREADS];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int row = blockIdx.x;
  const int64_t n = p.q_pos0 + row % p.n_q + 1;
  const int64_t n_cand = n - p.window;
  const int max_sel = p.window + p.topk;
  int32_t* out = p.idx + (int64_t)row * max_sel;
  if (n_cand <= p.topk) {  // every key 0..p is selected
    for (int j = tid; j < max_sel; j += SEL_THREADS) out[j] = j < n ? (int32_t)j : -1;
    if (tid == 0) p.count[row] = (int32_t)n;
    return;
  }
  const float* rowp = p.scores + (int64_t)row * p.ld_scores;
  const int nseg = (int)((n_cand + FR_SEG - 1) / FR_SEG);
  const int* cnt = ws.count + (int64_t)row * ws.nseg;
  int par = 0;
  // candidates kept over the whole row
  int64_t total = 0;
  for (int s0 = 0; s0 < nseg; s0 += SEL_THREADS) {
    int t;
    (void)block_excl_scan1(s0 + tid < nseg ? cnt[s0 + tid] : 0, tid, sh, par, t);
    total += t;
  }
  if (total >= p.topk && total <= FR_KCAP) {
    const uint32_t u_est = ws.u_est[row];
    int64_t placed = 0;
    for (int s0 = 0; s0 < nseg; s0 += SEL_THREADS) {
      const int c = s0 + tid < nseg ? cnt[s0 + tid] : 0;
      int t;
      const int before = block_excl_scan1(c, tid, sh, par, t);
      seg_cnt[tid] = c;
      seg_pos[tid] = (int)placed + before;
      __syncthreads();
      const int nb = min(SEL_THREADS, nseg - s0);
      // the stored candidates: a thread per kept position of the batch, the
      // segment found by a binary search of the positions, every load issued
      // before the first LDS write (one memory latency for the batch)
      constexpr int PER_T = FR_KCAP / SEL_THREADS;
      uint2 ev[PER_T];
      int dst[PER_T];
#pragma unroll
      for (int r = 0; r < PER_T; ++r) {
        const int j = tid + r * SEL_THREADS;   // position inside the batch
        dst[r] = -1;
        if (j < t) {
          int lo = 0, hi = nb - 1;   // the last segment that starts at or before j
          while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (seg_pos[mid] - (int)placed <= j) lo = mid; else hi = mid - 1;
          }
          if (seg_cnt[lo] <= FR_SCAP) {
            ev[r] = ws.kept[((int64_t)row * ws.nseg + s0 + lo) * FR_SCAP + (j - (seg_pos[lo] - (int)placed))];
            dst[r] = (int)placed + j;
          }
        }
      }
#pragma unroll
      for (int r = 0; r < PER_T; ++r) {
        if (dst[r] >= 0) {
          cval[dst[r]] = ev[r].x;
          cidx[dst[r]] = (int32_t)ev[r].y;
        }
      }
      for (int s = wv; s < nb; s += SEL_WAVES) {
        const int cs = seg_cnt[s], ps = seg_pos[s];
        if (cs > FR_SCAP) {
          // more than the slot holds: this wave compacts the segment again
          // from the row (the same candidates, the same order)
          const int64_t c0 = (int64_t)(s0 + s) * FR_SEG;
          const int64_t c1 = min(n_cand, c0 + FR_SEG);
          int wpos = ps;
          for (int64_t j0 = c0; j0 < c1; j0 += 4 * kWave) {
            const int64_t j = j0 + 4 * lane;
            uint32_t u4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) u4[e] = j + e < c1 ? fbits(rowp[j + e]) : 0u;
            uint64_t b4[4];
            int pp = wpos;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              b4[e] = __ballot(j + e < c1 && u4[e] >= u_est);
              pp += __builtin_amdgcn_mbcnt_hi((uint32_t)(b4[e] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b4[e], 0));
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if ((b4[e] >> lane) & 1) {
                cval[pp] = u4[e];
                cidx[pp] = (int32_t)(j + e);
                ++pp;
              }
              wpos += __popcll(b4[e]);
            }
          }
        }
      }
      placed += t;
      __syncthreads();
    }
    const int kept = (int)total;
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
    for (int j = tid; j < kept; j += SEL_THREADS) {
      kmin = min(kmin, cval[j]);
      kmax = max(kmax, cval[j]);
    }
    block_min_max(kmin, kmax, sh);
    pick_from_lds(cval, cidx, kept, kmin, kmax, p.topk, out, sh, par);
  } else {
    exact_row(rowp, n_cand, p.topk, out, sh, par);
  }
  for (int w = tid; w < p.window; w += SEL_THREADS) out[p.topk + w] = (int32_t)(n_cand + w);
  if (tid == 0) p.count[row] = max_sel;
}

bool select_few_rows(int B, int n_q, int64_t q_pos0, int window) {
  const int64_t max_cand = q_pos0 + n_q - window;
  return (int64_t)B * n_q <= FR_MAX_ROWS && max_cand >= FR_MIN_CAND;
}

size_t fr_layout(int rows, int64_t max_cand, char* base, FrWs* ws) {
  const int64_t nseg = (max_cand + FR_SEG - 1) / FR_SEG;
  auto a256 = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t est_bytes = a256((size_t)rows * 4);
  const size_t cnt_bytes = a256((size_t)rows * nseg * 4);
  const size_t kept_bytes = a256((size_t)rows * nseg * FR_SCAP * 8);
  if (ws) {
    ws->u_est = (uint32_t*)base;
    ws->count = (int*)(base + est_bytes);
    ws->kept = (uint2*)(base + est_bytes + cnt_bytes);
    ws->nseg = (int)nseg;
  }
  return est_bytes + cnt_bytes + kept_bytes;
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
  if (!select_few_rows(B, n_q, q_pos0, 1)) return 0;
  return fr_layout(B * n_q, q_pos0 + n_q - 1, nullptr, nullptr);
}

hipError_t launch_select(const SelectParams& p, void* ws_ptr, size_t /*ws_bytes*/, hipStream_t stream) {
  if (p.B * p.n_q == 0) return hipSuccess;
  if (!select_few_rows(p.B, p.n_q, p.q_pos0, p.window)) {
    hipLaunchKernelGGL(select_kernel, dim3((unsigned)(p.B * p.n_q)), dim3(SEL_THREADS), 0, stream, p);
    return hipGetLastError();
  }
  const int rows = p.B * p.n_q;
  FrWs ws;
  fr_layout(rows, p.q_pos0 + p.n_q - p.window, (char*)ws_ptr, &ws);
  hipLaunchKernelGGL(fr_compact_kernel, dim3((unsigned)ws.nseg, (unsigned)rows), dim3(SEL_THREADS), 0, stream, p, ws);
  hipLaunchKernelGGL(fr_final_kernel, dim3((unsigned)rows), dim3(SEL_THREADS), 0, stream, p, ws);
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

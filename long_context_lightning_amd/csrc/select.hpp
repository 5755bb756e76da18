// Exact top-k of the keys one workgroup holds: the threshold by three radix rounds in LDS, then
// the rank of every taken key in position order. Used by the selection inside the sparse-MLA
// launch.
//
// Selection rule of step 2 ("How GLM5.3 Sparse Attention Affects HBM Memory Usage", How it works
// / Model): the k largest scores, compared as reals, an equal score going to the lower position.
// Scores enter as order-preserving keys (score_key; -0.0 and +0.0 share a key, and no score
// gives key 0, which marks an absent position). Thread i holds PER keys of consecutive
// positions, thread i's before thread i+1's.
//   rounds: radix digits of the key (bits 31..21, 20..10, 9..0), each counted in a 2048-bin
//           LDS histogram over the keys that share the digits found so far, give the threshold
//           key (the k-th largest) and how many keys equal to it are taken. Every wave finds the
//           bin by itself (lane l sums 32 bins, a wave prefix sum picks the lane, then each lane
//           takes one of that lane's bins and a second prefix sum picks the bin), so a round
//           costs one barrier (round 0's histogram is counted by sel_count0 before the barrier
//           that precedes sel_threshold). Round 1 also records, per bin, whether its keys share
//           their low ten bits; when the chosen bin holds a single key value that value is the
//           threshold and round 2 is skipped (scores that differ in their top 22 key bits, e.g.
//           integers of magnitude below 2^14, never need it);
//   ranks:  each thread's taken keys as a bit mask (keys above the threshold, and of the keys
//           equal to it the first ones in position order, as many as are taken); workgroup
//           prefix sums of the counts above and equal give each thread the rank of its first
//           taken key.
// Subtractions are written so that none is guarded by a comparison (n - min(x, n), never
// x >= n ? 0 : n - x): the compiler marks a guarded one wrap-free, hoists it, and then folds
// comparisons and minima of its operands away.
#pragma once

#include "common.hpp"

namespace dsa {

constexpr int SEL_BINS = 2048;
// bin b is stored at word b + b / 32 (one pad word after every 32 bins, so that lane l reading
// the i-th bin of group l meets no other lane's bank), followed by one dummy bin per lane
constexpr int SEL_PADDED = SEL_BINS + SEL_BINS / 32;
constexpr int SEL_HIST = SEL_PADDED + WAVE;
constexpr int SEL_H1 = SEL_HIST;             // round 1's histogram (round 0's at word 0)
constexpr int SEL_LOW = 2 * SEL_HIST;        // round 1's low-bit summary per bin (see below)
constexpr int SEL_H2 = 3 * SEL_HIST;         // round 2's
constexpr int SEL_RED = 4 * SEL_HIST;        // [2][waves] prefix-sum partials
template <int THREADS>
constexpr int sel_scratch_words() { return SEL_RED + 2 * (THREADS / WAVE); }

__device__ __forceinline__ uint32_t sel_slot(uint32_t b) { return b + (b >> 5); }

// Taken-key mask of one thread.
template <int PER> struct SelMask { typedef uint32_t T; };
template <> struct SelMask<64> { typedef uint64_t T; };

__device__ __forceinline__ int sel_popc(uint32_t m) { return __popc(m); }
__device__ __forceinline__ int sel_popc(uint64_t m) { return __popcll(m); }
__device__ __forceinline__ uint32_t sel_top_bit(uint32_t m) { return 1u << (31 - __builtin_clz(m)); }
__device__ __forceinline__ uint64_t sel_top_bit(uint64_t m) {
  return 1ull << (63 - __builtin_clzll(m));
}
__device__ __forceinline__ int sel_low_index(uint32_t m) { return __builtin_ctz(m); }
__device__ __forceinline__ int sel_low_index(uint64_t m) { return __builtin_ctzll(m); }

// Loads PER scores, positions PER*tid .. PER*tid + PER - 1 of srow (positions at or past `lim`
// are left at 0; the keys mask them).
template <int PER>
__device__ __forceinline__ void sel_load_scores(const float* __restrict__ srow, int64_t lim,
                                                bool aligned, float (&v)[PER]) {
  const int64_t p0 = (int64_t)threadIdx.x * PER;
  if (aligned && p0 + PER <= lim) {
#pragma unroll
    for (int i = 0; i < PER / 4; ++i) {
      const f32x4 x = *(const f32x4*)(srow + p0 + 4 * i);
      v[4 * i] = x[0]; v[4 * i + 1] = x[1]; v[4 * i + 2] = x[2]; v[4 * i + 3] = x[3];
    }
  } else {
#pragma unroll
    for (int i = 0; i < PER; ++i) v[i] = p0 + i < lim ? srow[p0 + i] : 0.f;
  }
}

// Keys of this thread's scores; positions PER*tid + i at or past n are absent (0).
template <int PER>
__device__ __forceinline__ void sel_keys(const float (&v)[PER], int64_t n, uint32_t (&key)[PER]) {
  const int64_t p0 = (int64_t)threadIdx.x * PER;
#pragma unroll
  for (int i = 0; i < PER; ++i) key[i] = p0 + i < n ? score_key(v[i]) : 0u;
}

// Searches bins 0..2047 (bin b at word sel_slot(b)) from the top for the one holding the need-th
// largest key; every wave does it by itself and gets the same (bin, keys still needed inside it).
__device__ __forceinline__ void sel_find_bin(const uint32_t* __restrict__ hc, uint32_t need,
                                             uint32_t& bin, uint32_t& rem) {
  const int lane = lane_id();
  const int g = WAVE - 1 - lane;                         // this lane's bins 32g .. 32g + 31
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) sum += hc[33 * g + i];
  const uint32_t above = wave_incl_scan_u32(sum) - sum;  // keys in the bins of lower lanes
  const uint64_t hit = __ballot(above < need && above + sum >= need);
  const int fl = __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(hit));
  const uint32_t above_fl = __builtin_amdgcn_readlane(above, fl);
  // lane j (< 32) takes bin top - j of lane fl's 32 bins
  const int gf = WAVE - 1 - fl;
  const uint32_t h = lane < 32 ? hc[33 * gf + 31 - lane] : 0u;
  const uint32_t cum = above_fl + wave_incl_scan_u32(h) - h;
  const uint64_t hit2 = __ballot(cum < need && cum + h >= need);
  const int j = __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(hit2));
  bin = (uint32_t)(32 * gf + 31 - j);
  rem = need - min(__builtin_amdgcn_readlane(cum, j), need);
}

// Zeroes the first `hists` histograms of the scratch (round 0's, round 1's and the low-bit
// summaries are the first three; a barrier must follow before they are counted into).
template <int THREADS>
__device__ __forceinline__ void sel_clear(uint32_t* __restrict__ scratch, int hists) {
  for (int i = threadIdx.x; i < hists * SEL_HIST; i += THREADS) scratch[i] = 0;
}

// Counts round 0 (bits 31..21) into histogram 0, zeroed before a barrier; an absent key counts
// in its lane's dummy bin.
template <int PER>
__device__ __forceinline__ void sel_count0(const uint32_t (&key)[PER], uint32_t* __restrict__ h0) {
  const int lane = lane_id();
#pragma unroll
  for (int i = 0; i < PER; ++i) atomicAdd(&h0[key[i] ? sel_slot(key[i] >> 21) : SEL_PADDED + lane], 1u);
}

struct SelThreshold {
  uint32_t thr;     // the k-th largest key
  uint32_t need;    // keys equal to thr that are taken (the first ones in position order)
  uint32_t bin0;    // round 0's bin of thr
  uint32_t need0;   // keys taken from bin0 (every key in a higher bin is taken)
};

// The threshold of the workgroup's keys for k (at least k keys present). Histogram 0 holds round
// 0's counts and was published by a barrier; histogram 1 and the low-bit summaries are zero. One
// or two barriers: round 1 also ORs, per fine bin, the low ten bits of each key and their
// complement into one word, so that when the chosen fine bin holds a single key value (its keys'
// low bits OR to a value disjoint from their complements' OR) that value is the threshold and
// round 2 is skipped.
template <int THREADS, int PER>
__device__ __forceinline__ SelThreshold sel_threshold(const uint32_t (&key)[PER], uint32_t k,
                                                      uint32_t* __restrict__ scratch) {
  SelThreshold r;
  uint32_t need = k, bin;
  sel_find_bin(scratch, need, bin, need);
  r.bin0 = bin;
  r.need0 = need;
  uint32_t pref = bin;                         // bits 31..21 of the threshold
  // round 1: bits 20..10 of the keys sharing them (H1; H2 is cleared meanwhile)
  {
    uint32_t* hc = scratch + SEL_H1;
    for (int i = threadIdx.x; i < SEL_HIST; i += THREADS) scratch[SEL_H2 + i] = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if ((key[i] >> 21) == pref) {
        const uint32_t sl = sel_slot((key[i] >> 10) & 2047u);
        atomicAdd(&hc[sl], 1u);
        atomicOr(&scratch[SEL_LOW + sl], (key[i] & 1023u) | ((~key[i] & 1023u) << 10));
      }
    __syncthreads();
    sel_find_bin(hc, need, bin, need);
  }
  pref = (pref << 11) | bin;                   // bits 31..10
  {
    const uint32_t lo = scratch[SEL_LOW + sel_slot(bin)];
    if (((lo & 1023u) & (lo >> 10)) == 0) {   // uniform: one key value in the chosen bin
      r.thr = (pref << 10) | (lo & 1023u);
      r.need = need;
      return r;
    }
  }
  // round 2: bits 9..0 (H2; bins 1024.. stay empty)
  {
    uint32_t* hc = scratch + SEL_H2;
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if ((key[i] >> 10) == pref) atomicAdd(&hc[sel_slot(key[i] & 1023u)], 1u);
    __syncthreads();
    sel_find_bin(hc, need, bin, need);
  }
  r.thr = (pref << 10) | bin;
  r.need = need;
  return r;
}

// This thread's taken keys (exactly the k of sel_threshold over the workgroup) as a mask over its
// PER keys, and the rank in position order of its first taken key: every key above the
// threshold, and the first s.need keys equal to it in position order (the count of keys above it
// is k - s.need). The counts above and equal meet in one exchange of wave totals. red: 2 * waves
// words of scratch that no other code reads meanwhile. One barrier.
template <int THREADS, int PER>
__device__ __forceinline__ void sel_ranks(const uint32_t (&key)[PER], const SelThreshold& s,
                                          uint32_t* __restrict__ red,
                                          typename SelMask<PER>::T& taken, uint32_t& before) {
  typedef typename SelMask<PER>::T M;
  constexpr int NW = THREADS / WAVE;
  const int wave = threadIdx.x / WAVE, lane = lane_id();
  const uint32_t thr = s.thr, need = s.need;
  M gt = 0, eq = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    gt |= (key[i] > thr ? (M)1 : (M)0) << i;
    eq |= (key[i] == thr ? (M)1 : (M)0) << i;
  }
  const uint32_t cg = sel_popc(gt), ce = sel_popc(eq);
  const uint32_t ig = wave_incl_scan_u32(cg), ie = wave_incl_scan_u32(ce);
  if (lane == WAVE - 1) {
    red[wave] = ig;
    red[NW + wave] = ie;
  }
  __syncthreads();
  uint32_t g_before = ig - cg, e_before = ie - ce;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    g_before += w < wave ? red[w] : 0u;
    e_before += w < wave ? red[NW + w] : 0u;
  }
  // equal keys taken before this thread, and this thread's: its lowest positions
  const uint32_t e_taken_before = min(e_before, need);
  uint32_t drop = ce - min(ce, need - e_taken_before);
  while (drop > 0) {                           // clear the highest equal positions
    eq ^= sel_top_bit(eq);
    --drop;
  }
  taken = gt | eq;
  before = g_before + e_taken_before;
}

}  // namespace dsa

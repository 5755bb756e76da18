// Causal per-query top-k ("How GLM5.3 Sparse Attention Affects HBM Memory Usage", How it works /
// Model: top-k 2048, dense below 2K visible tokens, one selection shared by all heads).
//
// Selection rule: the k largest scores among positions 0..p, scores compared as reals
// (-0.0 == +0.0), an equal score going to the lower position; output ascending, -1 padded.
// Scores are finite or infinite; a NaN score is never selected.
//
// Batches of many rows (prefill, wide decode) use one workgroup of 1024 threads per query row,
// described here; batches of a few long rows split each row over several workgroups (further
// down). With one workgroup per row the scores stay in registers:
//   * the row is cut into chunks of UNITS*4096 positions (UNITS <= 8) held in registers. A row
//     of one chunk gives each lane UNITS consecutive 16-byte groups (consecutive positions);
//     longer rows keep a unit-major layout, lane l of wave w's slice holding groups u*64 + l.
//     A row of one chunk is read from memory once. A longer row is streamed once when k fits
//     the candidate buffer (after each chunk only the top k of candidates and chunk survive,
//     in LDS); otherwise its chunks are re-read on every pass. Slots outside the row hold NaN,
//     which no comparison or bin counts;
//   * round 0 histograms every score into 2048 bins linear in the value between the row's
//     smallest and largest score. If the bin holding the k-th largest score has at most 64
//     scores, one wave ranks them directly. Otherwise round 1 splits that bin into 2048 finer
//     linear bins, and later rounds split the chosen bin in the space of order-preserving
//     32-bit keys into bins of a power-of-two width (at most three such rounds reach one key).
//     Bin indices are monotone functions of the score (a rounded fused multiply-add, clamped
//     and truncated), so every bin is a contiguous range of scores. From round 1 on each bin
//     also records its smallest and largest key. The bin holding the k-th largest score is found
//     with DPP wave prefix sums and one exchange of wave totals. The select ends when the scores
//     still needed from the chosen bin are all of its scores (everything at or above its
//     smallest score is taken) or when the bin holds a single value. The result is a threshold
//     score T and a count `need`: a position is selected if its score is above T, or equal to T
//     and among the first `need` such positions;
//   * compaction in index order: for a row of one chunk each lane counts its scores above and
//     equal to T, wave prefix sums and one exchange of wave totals give the counts before it,
//     and the lane stores its taken positions straight to their output slots; for longer rows
//     the per-wave counts (ballot popcounts) are exchanged once per chunk, and inside the wave
//     each step of 256 positions ranks its taken positions with lane-mask counts.
#include <algorithm>

#include <map>
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"

namespace dsa {
namespace {

constexpr int TK_THREADS = 1024;
constexpr int TK_WAVES = TK_THREADS / WAVE;
constexpr int TK_BINS = 2048;
constexpr int TK_HIST = TK_BINS + 64;          // bin TK_BINS collects NaN (never selected)
constexpr int TK_OBUF = 2048;                  // k up to this is staged in LDS

// The score whose key is k (inverse of score_key).
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

struct MinF32 {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const {
    return __float_as_uint(fminf(__uint_as_float(a), __uint_as_float(b)));
  }
};
struct MaxF32 {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const {
    return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
  }
};

struct TopkShared {
  uint32_t hist[2][TK_HIST];           // counts, alternating between rounds
  uint32_t bmin[2][TK_BINS];           // smallest / largest key per bin (rounds after the first)
  uint32_t bmax[2][TK_BINS];
  uint32_t red_a[TK_WAVES];            // wave exchanges of the select
  uint32_t red_b[TK_WAVES];
  uint32_t red_c[TK_WAVES];            // wave exchanges of the compaction
  uint32_t red_d[TK_WAVES];
  uint32_t sel_bin, sel_need, sel_count, sel_min, sel_max;
  // scores of a round-0 bin with at most WAVE entries (NaN past the count), ranked by one wave
  __attribute__((aligned(16))) float few[WAVE];
  uint32_t few_n, few_need;
  float few_thr;
  // selected positions, written out coalesced at the end; the last WAVE entries take the
  // writes of lanes whose element is not selected (one per lane, so no store needs a branch)
  int32_t obuf[TK_OBUF + WAVE];
  float cand_val[TK_OBUF];             // candidates of a streamed row (scores, positions)
  int32_t cand_pos[TK_OBUF];
};

// Finds, in histogram h (bins BPT*tid .. BPT*tid + BPT - 1 per thread, BPT = TK_BINS / THREADS,
// keys counted from the top bin down), the bin holding the need-th largest key, and publishes it
// with the keys still needed from it, its count and its smallest and largest key. Two barriers;
// all threads must call.
template <int THREADS>
__device__ __forceinline__ void select_bin(const uint32_t* h, const uint32_t* bmin,
                                           const uint32_t* bmax, uint32_t need,
                                           TopkShared& sh) {
  constexpr int BPT = TK_BINS / THREADS;
  static_assert(BPT * THREADS == TK_BINS, "whole bins per thread");
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  uint32_t hv[BPT];
  uint32_t sum = 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    hv[j] = h[BPT * tid + j];
    sum += hv[j];
  }
  const uint32_t incl = wave_incl_scan_u32(sum);
  const uint32_t wave_tot = last_lane(incl);
  if (lane_id() == 0) sh.red_a[wave] = wave_tot;
  __syncthreads();
  uint32_t above = wave_tot - incl;            // keys in bins above this thread's bins
#pragma unroll
  for (int w = 0; w < THREADS / WAVE; ++w)
    if (w > wave) above += sh.red_a[w];
  int b = -1;
#pragma unroll
  for (int j = BPT - 1; j >= 0; --j) {         // this thread's bins from the top
    if (b < 0 && above < need && above + hv[j] >= need) {
      b = BPT * tid + j;
      sh.sel_need = need - above;
      sh.sel_count = hv[j];
    }
    above += hv[j];
  }
  if (b >= 0) {
    sh.sel_bin = b;
    sh.sel_min = bmin[b];
    sh.sel_max = bmax[b];
  }
  __syncthreads();
}

// Bin of x under x -> clamp(trunc(fma(x, scale, bias)), 0, TK_BINS-1), monotone in x for a finite
// scale >= 0 and finite bias; a NaN x goes to the extra bin TK_BINS.
__device__ __forceinline__ uint32_t lin_bin(float x, float scale, float bias) {
  const float f = fminf(__builtin_fmaf(x, scale, bias), (float)(TK_BINS - 1));
  return x == x ? (uint32_t)fmaxf(f, 0.f) : (uint32_t)TK_BINS;
}

// MODE: 0 = every row fits one register chunk; 1 = longer rows streamed through the candidate
// buffer (k <= TK_OBUF); 2 = longer rows re-read chunk by chunk on every pass.
template <int THREADS, int UNITS, int MODE>
__global__ __launch_bounds__(THREADS, 4) void topk_rows(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ cu_q,
    const int64_t* __restrict__ cu_k, int nseq, int total_q, int64_t total_k, int k,
    int32_t* __restrict__ out) {
  __shared__ TopkShared sh;
  constexpr int SLICE4 = UNITS * WAVE;           // 16-byte groups per wave and chunk
  constexpr int CHUNK4 = UNITS * THREADS;     // 16-byte groups per chunk
  constexpr uint32_t ALL = 0xffffffffu;

  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  const float* srow = scores + (int64_t)t * ld;
  // The row is read in aligned 16-byte groups; `off` floats of the first group precede it.
  // For the first row of a score matrix that does not start on a 16-byte boundary, and the
  // last row of one that does not end on one, an edge group reaches up to 12 bytes outside the
  // buffer, but only inside the aligned 16 bytes that also hold a buffer element, so never
  // into another page; the positions outside the row are masked before use. Reading those
  // groups element by element instead makes the compiler wait for every outstanding load at
  // each use, which costs the split top-k about 6 us per call.
  // Positions fit in 32 bits (they are stored as int32).
  const int off = (int)((reinterpret_cast<uintptr_t>(srow) >> 2) & 3);
  const f32x4* g4 = reinterpret_cast<const f32x4*>(srow - off);
  // Single-chunk rows (MODE 0) give each lane UNITS consecutive groups, so its elements are
  // consecutive positions and the compaction is one in-order walk per lane; longer rows keep
  // the unit-major layout (each load instruction reads 64 consecutive groups).
  constexpr bool contiguous = MODE == 0;
  constexpr int USTEP = contiguous ? 1 : WAVE;   // group distance of a lane's units
  const int lane_g = wave * SLICE4 + lane * (contiguous ? UNITS : 1);   // unit 0, chunk 0
  const float qnan = __uint_as_float(0x7fc00000u);
  // If the row's whole allocated span fits one register chunk, its loads go out before the
  // sequence lookup (the row's address does not depend on it) and the visible length masks
  // the values afterwards.
  const int ng4_span = (int)((ld + off + 3) >> 2);
  const bool early = ng4_span <= CHUNK4;
  f32x4 pre[UNITS];
  if (early) {
#pragma unroll
    for (int u = 0; u < UNITS; ++u) {
      const int g = lane_g + u * USTEP;
      pre[u] = g < ng4_span ? g4[g] : f32x4{qnan, qnan, qnan, qnan};
    }
  }
  const QueryPos qp = query_pos(cu_q, cu_k, nseq, total_k, t);
  const int64_t n = min(qp.p + 1, ld);           // visible positions 0..n-1 (0 if invalid)
  int32_t* orow = out + (int64_t)t * k;
  if (n <= k) {                                  // dense path: everything visible is selected
    for (int i = tid; i < k; i += THREADS) orow[i] = i < n ? i : -1;
    return;
  }
  const int ni = (int)n;
  const int ng4 = (ni + off + 3) >> 2;
  const int nchunks = (ng4 + CHUNK4 - 1) / CHUNK4;

  float x[UNITS][4];
  // Unit u of this lane in chunk c is group c*CHUNK4 + lane_g + USTEP*u; its element e is
  // position 4*group + e - off.
  auto load_chunk = [&](int c) {
#pragma unroll
    for (int u = 0; u < UNITS; ++u) {
      const int g = c * CHUNK4 + lane_g + u * USTEP;
      f32x4 v = {qnan, qnan, qnan, qnan};
      if (g < ng4) v = g4[g];
#pragma unroll
      for (int e = 0; e < 4; ++e) x[u][e] = v[e];
      if (g == 0 || g == ng4 - 1) {              // the row's first and last groups may be partial
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int pos = 4 * g + e - off;
          if (pos < 0 || pos >= ni) x[u][e] = qnan;
        }
      }
    }
  };
  if (early) {
#pragma unroll
    for (int u = 0; u < UNITS; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int pos = 4 * (lane_g + u * USTEP) + e - off;
        x[u][e] = (pos >= 0 && pos < ni) ? pre[u][e] : qnan;
      }
  } else {
    load_chunk(0);
  }

  // Rows longer than one chunk are streamed when k fits the candidate buffer: after each chunk
  // only the top k of (earlier candidates, chunk) survive, ties at the threshold keeping their
  // lowest positions, which is exactly the part of them the final selection can take. Thread i
  // holds candidates CPT*i.. in index order (NaN past the count). Otherwise every pass re-reads
  // the row chunk by chunk.
  constexpr int CPT = TK_OBUF / THREADS;
  constexpr bool stream = MODE == 1;
  constexpr bool resident = MODE != 2;           // x holds the whole current segment
  float cv[CPT];
  int32_t cp[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) { cv[j] = qnan; cp[j] = 0; }

  // f(v) for every score of the current segment
  auto visit = [&](auto&& f) {
    auto regs = [&]() {
#pragma unroll
      for (int u = 0; u < UNITS; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) f(x[u][e]);
    };
    if constexpr (resident) {
      regs();
      if constexpr (stream)
#pragma unroll
        for (int j = 0; j < CPT; ++j) f(cv[j]);
    } else {
      for (int c = 0; c < nchunks; ++c) {
        load_chunk(c);
        regs();
      }
    }
  };

  // The threshold T of the current segment and how many scores equal to T are taken (all of
  // them when the result is ALL).
  auto select = [&](float& thr, uint32_t& thr_need) {
    for (int i = tid; i < TK_HIST; i += THREADS) {
      sh.hist[0][i] = 0;
      sh.hist[1][i] = 0;
    }
    for (int i = tid; i < TK_BINS; i += THREADS) {
      sh.bmin[0][i] = ALL;
      sh.bmin[1][i] = ALL;
      sh.bmax[0][i] = 0u;
      sh.bmax[1][i] = 0u;
    }
    if (tid < WAVE) sh.few[tid] = qnan;
    if (tid == 0) sh.few_n = 0;
    // value range (fminf / fmaxf skip NaN)
    float xmin = __int_as_float(0x7f800000), xmax = -xmin;
    visit([&](float v) {
      xmin = fminf(xmin, v);
      xmax = fmaxf(xmax, v);
    });
    xmin = __uint_as_float(last_lane(wave_incl_scan(__float_as_uint(xmin), 0x7f800000u, MinF32())));
    xmax = __uint_as_float(last_lane(wave_incl_scan(__float_as_uint(xmax), 0xff800000u, MaxF32())));
    if (lane == 0) { sh.red_a[wave] = __float_as_uint(xmin); sh.red_b[wave] = __float_as_uint(xmax); }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < (THREADS / WAVE); ++w) {
      xmin = fminf(xmin, __uint_as_float(sh.red_a[w]));
      xmax = fmaxf(xmax, __uint_as_float(sh.red_b[w]));
    }

    uint32_t need = (uint32_t)k;                 // scores to take from the current range
    thr = xmin;
    thr_need = need;
    if (!(xmin < xmax)) return;                  // a single value: take k of them
    // round 0: linear bins over [xmin, xmax]
    const float s0 = (float)TK_BINS / (xmax - xmin);
    uint32_t lo, hi, count;
    if (s0 > 0.f && s0 <= __FLT_MAX__) {         // finite range: xmin and xmax are finite
      const float c0 = -xmin * s0;
      visit([&](float v) {
        if (v == v) atomicAdd(&sh.hist[0][lin_bin(v, s0, c0)], 1u);
      });
      __syncthreads();
      select_bin<THREADS>(sh.hist[0], sh.bmin[0], sh.bmax[0], need, sh);
      const uint32_t bin0 = sh.sel_bin;
      need = sh.sel_need;
      if (sh.sel_count <= (uint32_t)WAVE) {
        // Few scores in bin0: they go to LDS and one wave ranks them. The need-th largest is
        // the threshold; of the scores equal to it, those not counted above it are taken.
        visit([&](float v) {
          if (lin_bin(v, s0, c0) == bin0) sh.few[atomicAdd(&sh.few_n, 1u)] = v;
        });
        __syncthreads();
        if (wave == 0) {
          const float v = sh.few[lane];
          uint32_t gt = 0, eq = 0;
#pragma unroll
          for (int j = 0; j < WAVE / 4; ++j) {
            const f32x4 u = reinterpret_cast<const f32x4*>(sh.few)[j];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              gt += u[e] > v ? 1u : 0u;
              eq += u[e] == v ? 1u : 0u;
            }
          }
          if (gt < need && need <= gt + eq) {    // NaN entries have eq = 0
            sh.few_thr = v;
            sh.few_need = need - gt;
          }
        }
        __syncthreads();
        thr = sh.few_thr;
        thr_need = sh.few_need;
        return;
      }
      // round 1: the scores of bin0, in 2048 linear sub-bins with their smallest and largest key
      float s1 = s0 * (float)TK_BINS;
      float c1 = -(xmin + (float)bin0 / s0) * s1;
      if (!(s1 <= __FLT_MAX__ && c1 <= __FLT_MAX__ && c1 >= -__FLT_MAX__)) { s1 = 0.f; c1 = 0.f; }
      for (int i = tid; i < TK_HIST; i += THREADS) sh.hist[0][i] = 0;  // read in select_bin
      visit([&](float v) {
        if (lin_bin(v, s0, c0) == bin0) {
          const uint32_t b = lin_bin(v, s1, c1);
          const uint32_t kk = score_key(v);
          atomicAdd(&sh.hist[1][b], 1u);
          atomicMin(&sh.bmin[1][b], kk);
          atomicMax(&sh.bmax[1][b], kk);
        }
      });
      __syncthreads();
      select_bin<THREADS>(sh.hist[1], sh.bmin[1], sh.bmax[1], need, sh);
      lo = sh.sel_min;
      hi = sh.sel_max;
      count = sh.sel_count;
      need = sh.sel_need;
    } else {                                     // an infinite score, or a denormal-wide range
      lo = score_key(xmin);
      hi = score_key(xmax);
      count = ALL;
    }
    // later rounds: keys [lo, hi] of the chosen bin, bins of a power-of-two width
    for (int r = 2;; ++r) {
      if (count == need) {                       // the whole bin is taken: scores >= its minimum
        thr = key_value(lo);
        thr_need = ALL;
        break;
      }
      if (lo == hi) {                            // one value left: take `need` of them
        thr = key_value(lo);
        thr_need = need;
        break;
      }
      const uint32_t span = hi - lo;
      int shift = 0;
      while ((span >> shift) >= (uint32_t)TK_BINS) ++shift;
      const int cur = r & 1;
      uint32_t* hc = sh.hist[cur];
      uint32_t* mn = sh.bmin[cur];
      uint32_t* mx = sh.bmax[cur];
      // the other buffers were last read in the previous select_bin; cleared for the next round
      for (int i = tid; i < TK_BINS; i += THREADS) {
        sh.hist[cur ^ 1][i] = 0;
        sh.bmin[cur ^ 1][i] = ALL;
        sh.bmax[cur ^ 1][i] = 0u;
      }
      const float vlo = key_value(lo), vhi = key_value(hi);
      visit([&](float v) {
        if (v >= vlo && v <= vhi) {
          const uint32_t kk = score_key(v);
          const uint32_t b = (kk - lo) >> shift;
          atomicAdd(&hc[b], 1u);
          atomicMin(&mn[b], kk);
          atomicMax(&mx[b], kk);
        }
      });
      __syncthreads();
      select_bin<THREADS>(hc, mn, mx, need, sh);
      count = sh.sel_count;
      need = sh.sel_need;
      lo = sh.sel_min;
      hi = sh.sel_max;
    }
  };

  // Compaction in index order: a position is taken if its score is above thr, or equal to it
  // and among the first thr_need such positions; the slot of a taken position is the number of
  // positions taken before it. sink(take, slot, position, score) stores a position: a taken one
  // at its slot, any other (the branch-free walk of single-chunk rows) at the lane's spare entry.
  // The candidates of a streamed row come first (all their positions precede the chunk's).
  auto compact_cands = [&](float thr, uint32_t thr_need, uint32_t& gt_tot, uint32_t& eq_tot,
                           auto&& sink) {
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      gt += cv[j] > thr;
      eq += cv[j] == thr;
    }
    const uint32_t igt = wave_incl_scan_u32(gt), ieq = wave_incl_scan_u32(eq);
    if (lane == WAVE - 1) { sh.red_c[wave] = igt; sh.red_d[wave] = ieq; }
    __syncthreads();
    uint32_t gt_b = igt - gt, eq_b = ieq - eq;
    gt_tot = 0;
    eq_tot = 0;
#pragma unroll
    for (int w = 0; w < (THREADS / WAVE); ++w) {
      const uint32_t a = sh.red_c[w], b = sh.red_d[w];
      if (w < wave) { gt_b += a; eq_b += b; }
      gt_tot += a;
      eq_tot += b;
    }
    __syncthreads();                             // red_c / red_d are reused by the chunk
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      if (cv[j] > thr) {
        sink(true, gt_b + min(eq_b, thr_need), cp[j], cv[j]);
        ++gt_b;
      } else if (cv[j] == thr) {
        if (eq_b < thr_need) sink(true, gt_b + eq_b, cp[j], cv[j]);
        ++eq_b;
      }
    }
  };
  // chunk c (x holding it); gt_chunk / eq_chunk count the scores above / equal to thr before it
  auto compact_chunk = [&](int c, float thr, uint32_t thr_need, uint32_t& gt_chunk,
                           uint32_t& eq_chunk, auto&& sink) {
    if constexpr (contiguous) {
      // Each lane counts its own elements; wave prefix sums and one exchange of wave totals
      // give the counts before each lane, which then walks its consecutive positions in order
      // (a taken position's slot is the number of positions taken before it).
      uint32_t gt = 0, eq = 0;
#pragma unroll
      for (int u = 0; u < UNITS; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          gt += x[u][e] > thr;
          eq += x[u][e] == thr;
        }
      const uint32_t igt = wave_incl_scan_u32(gt), ieq = wave_incl_scan_u32(eq);
      if (lane == WAVE - 1) { sh.red_c[wave] = igt; sh.red_d[wave] = ieq; }
      __syncthreads();
      uint32_t gt_b = gt_chunk + igt - gt, eq_b = eq_chunk + ieq - eq;
#pragma unroll
      for (int w = 0; w < (THREADS / WAVE); ++w) {
        const uint32_t a = sh.red_c[w], b = sh.red_d[w];
        if (w < wave) { gt_b += a; eq_b += b; }
        gt_chunk += a;
        eq_chunk += b;
      }
      const int p0 = 4 * (c * CHUNK4 + lane_g) - off;
#pragma unroll
      for (int u = 0; u < UNITS; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = x[u][e];
          const bool above = v > thr, equal = v == thr;
          const uint32_t slot = gt_b + (above ? min(eq_b, thr_need) : eq_b);
          sink((above || (equal && eq_b < thr_need)) && slot < (uint32_t)k, slot,
               p0 + 4 * u + e, v);
          gt_b += above;
          eq_b += equal;
        }
    } else {
    uint32_t gt = 0, eq = 0;
#pragma unroll
      for (int u = 0; u < UNITS; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          gt += (uint32_t)__popcll(__ballot(x[u][e] > thr));
          eq += (uint32_t)__popcll(__ballot(x[u][e] == thr));
        }
      if (lane == 0) { sh.red_c[wave] = gt; sh.red_d[wave] = eq; }
      __syncthreads();
      uint32_t gt_before = gt_chunk, eq_before = eq_chunk;
#pragma unroll
      for (int w = 0; w < (THREADS / WAVE); ++w) {
        const uint32_t a = sh.red_c[w], b = sh.red_d[w];
        if (w < wave) { gt_before += a; eq_before += b; }
        gt_chunk += a;
        eq_chunk += b;
      }
      __syncthreads();                             // red_c / red_d are reused by the next chunk
      uint32_t eqc = eq_before;                    // equal scores before the current step
      uint32_t base = gt_before + min(eq_before, thr_need);  // output slot of the step's first take
#pragma unroll
      for (int u = 0; u < UNITS; ++u) {
        // step u covers positions (lane, e) in lane-major order
        uint64_t tm[4];
        uint64_t eq_any = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          tm[e] = __ballot(x[u][e] > thr);
          eq_any |= __ballot(x[u][e] == thr);
        }
        if (eq_any) {                              // some scores equal thr: rank them
          uint64_t qm[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) qm[e] = __ballot(x[u][e] == thr);
          uint32_t rank = eqc;
#pragma unroll
          for (int e = 0; e < 4; ++e) rank += lanes_below(qm[e]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool is_eq = x[u][e] == thr;
            tm[e] |= __ballot(is_eq && rank < thr_need);
            rank += is_eq;
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) eqc += (uint32_t)__popcll(qm[e]);
        }
        uint32_t slot = base;
#pragma unroll
        for (int e = 0; e < 4; ++e) slot += lanes_below(tm[e]);
        const int p0 = 4 * (c * CHUNK4 + lane_g + u * USTEP) - off;
        const uint64_t lane_bit = 1ull << lane;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (tm[e] & lane_bit) {
            if (slot < (uint32_t)k) sink(true, slot, p0 + e, x[u][e]);
            ++slot;
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) base += (uint32_t)__popcll(tm[e]);
      }
    }
  };

  // Streamed rows with k <= TK_OBUF stage the output in LDS (every slot starts at -1) and
  // write it out with coalesced stores at the end. Single-chunk rows store each selected
  // position straight to memory: a lane's positions go to consecutive slots, and with n > k
  // exactly k are selected, so every slot is written.
  const bool staged = MODE != 0 && k <= TK_OBUF;
  auto out_sink = [&](bool take, uint32_t slot, int pos, float) {
    if (staged) sh.obuf[take ? slot : TK_OBUF + lane] = pos;
    else if (take) orow[slot] = pos;
  };
  if (staged)
    for (int i = tid; i < k; i += THREADS) sh.obuf[i] = -1;

  float thr = 0.f;
  uint32_t thr_need;
  if constexpr (stream) {
    for (int c = 0; c < nchunks; ++c) {
      if (c > 0) {
        // The k candidates are all >= the previous threshold, and a later score equal to it
        // loses the tie to every candidate of that value: only scores above it can still be
        // taken, so the rest are masked out of every pass of this segment.
        const float prev = thr;
        load_chunk(c);
#pragma unroll
        for (int u = 0; u < UNITS; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (!(x[u][e] > prev)) x[u][e] = qnan;
      }
      select(thr, thr_need);
      uint32_t gt_tot = 0, eq_tot = 0;
      if (c + 1 < nchunks) {                     // the segment's top k become the candidates
        auto cand_sink = [&](bool, uint32_t slot, int pos, float v) {
          sh.cand_val[slot] = v;
          sh.cand_pos[slot] = pos;
        };
        if (c > 0) compact_cands(thr, thr_need, gt_tot, eq_tot, cand_sink);
        compact_chunk(c, thr, thr_need, gt_tot, eq_tot, cand_sink);
        __syncthreads();
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
          const int i = CPT * tid + j;
          cv[j] = i < k ? sh.cand_val[i] : qnan;
          cp[j] = i < k ? sh.cand_pos[i] : 0;
        }
        __syncthreads();                         // the buffer is rewritten by the next segment
      } else {
        compact_cands(thr, thr_need, gt_tot, eq_tot, out_sink);
        compact_chunk(c, thr, thr_need, gt_tot, eq_tot, out_sink);
      }
    }
  } else {
    select(thr, thr_need);
    uint32_t gt_chunk = 0, eq_chunk = 0;         // scores above / equal to thr in earlier chunks
    if constexpr (MODE == 0) {
      compact_chunk(0, thr, thr_need, gt_chunk, eq_chunk, out_sink);
    } else {
      for (int c = 0; c < nchunks; ++c) {
        load_chunk(c);
        compact_chunk(c, thr, thr_need, gt_chunk, eq_chunk, out_sink);
      }
    }
  }
  if (staged) {
    __syncthreads();
    // non-temporal: read by the next launch, so not left dirty in L2 at this one's end
    for (int i = tid; i < k; i += THREADS) __builtin_nontemporal_store(sh.obuf[i], orow + i);
  }
}

// ---------------------------------------------------------------------------------------------
// Rows split over several workgroups. A batch of a few long rows (long-context decode) leaves
// most compute units idle under one workgroup per row, so each row is cut into chunks of
// SP_CHUNK positions, one 256-thread workgroup per chunk with the chunk in registers. The
// workgroups of a row meet through per-row state in the workspace.
//
// One launch (rows of at most 256 chunks, topk_split_fused): the state is zero-filled first (by
// the decode indexer of the same step, or by a small launch of its own), then the workgroups of
// a row meet at three row barriers (device-scope counters and release words, bounded polls):
//   1  round-0 histogram: 2048 bins of the order-preserving key's top 11 bits, added into the
//      row's histogram with one global atomic per non-empty bin
//   2  the bin holding the k-th largest score split by the next 11 key bits (counts only)
//   3  per chunk, the scores above the chosen fine bin and inside it; when the chosen bin is
//      neither taken whole nor one value, the positions inside it are appended to a per-row
//      candidate list
//   4  every workgroup resolves the threshold (from the candidates when needed, in key space),
//      sums the counts of the chunks before its own and writes its selected positions in
//      index order.
// Five launches (longer rows), whose boundaries order everything:
//   prep     chunk minimum / maximum; clears the row's histograms
//   hist0    2048 bins linear between the row's smallest and largest score (bins of a
//            power-of-two key width when that range is not finite)
//   hist1    the bin holding the k-th largest score split into 2048 finer bins, with each
//            bin's smallest and largest key
//   count    as phase 3 above
//   compact  as phase 4 above.
// Every workgroup of a row derives the same bins from the same global values, so they agree on
// every decision.
// ---------------------------------------------------------------------------------------------
constexpr int SP_THREADS = 256;
constexpr int SP_WAVES = SP_THREADS / WAVE;
constexpr int SP_UNITS = 8;
constexpr int SP_SLICE4 = SP_UNITS * WAVE;          // 16-byte groups per wave and chunk
constexpr int SP_CHUNK4 = SP_UNITS * SP_THREADS;    // 16-byte groups per chunk (8192 positions)
constexpr int SP_BPT = TK_BINS / SP_THREADS;        // bins per thread in a select

// Per-row words of the workspace.
constexpr int RW_HIST0 = 0;
constexpr int RW_HIST1 = TK_BINS;
constexpr int RW_MIN1 = 2 * TK_BINS;
constexpr int RW_MAX1 = 3 * TK_BINS;
constexpr int RW_CAND_N = 4 * TK_BINS;
// Row barrier words of the one-launch path, 256 bytes apart: arrivals of the chunks c with
// c % 8 == g (8 words), arrivals of completed groups, then the round each group may pass (8).
constexpr int RW_BAR = 4 * TK_BINS + 64;
constexpr int BAR_STRIDE = 64;
constexpr int RW_WORDS = RW_BAR + 17 * BAR_STRIDE;

struct SplitWs {
  uint32_t* rows;      // [total_q][RW_WORDS]
  float2* minmax;      // [total_q][max_chunks]  chunk min / max score
  uint2* counts;       // [total_q][max_chunks]  chunk (above, inside) the chosen fine bin
  uint32_t* cand;      // [total_q][cand_cap]    positions inside the chosen fine bin
  uint32_t* candk;     // [total_q][cand_cap]    their keys
  int max_chunks;
  int max_k;
  int64_t cand_cap;
};

struct SplitShared {
  uint32_t hist[TK_BINS];
  uint32_t bmin[TK_BINS];
  uint32_t bmax[TK_BINS];
  uint32_t red_a[SP_WAVES], red_b[SP_WAVES], red_c[SP_WAVES], red_d[SP_WAVES];
  uint32_t sel_bin, sel_need, sel_count, sel_min, sel_max, bcast;
};

// Row t, chunk c of this workgroup and the chunk's place in the score row.
struct SplitChunk {
  int t, c;
  int ni;                 // visible positions 0..ni-1
  int off, ng4, nchunks;  // the row is read in aligned 16-byte groups; `off` floats precede it
  bool dense;             // ni <= k: everything visible is selected
  const float* srow;
  const f32x4* g4;
};

// Workspace words that other workgroups of the same launch write (the one-launch path below)
// are accessed with relaxed device-scope atomics: an atomic load or store at agent scope is
// served by the device's coherence point, not by a copy in one XCD's L2, so it sees what a
// workgroup on another XCD wrote once that workgroup's operation has completed. COH = false is
// an ordinary access (the five-launch path, where a launch boundary orders everything).
template <bool COH>
__device__ __forceinline__ uint32_t ws_ld(const uint32_t* p) {
  if constexpr (COH) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else return *p;
}
template <bool COH>
__device__ __forceinline__ void ws_st(uint32_t* p, uint32_t v) {
  if constexpr (COH) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}
template <bool COH>
__device__ __forceinline__ uint64_t ws_ld64(const uint64_t* p) {
  if constexpr (COH) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else return *p;
}
template <bool COH>
__device__ __forceinline__ void ws_st64(uint64_t* p, uint64_t v) {
  if constexpr (COH) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}

// Bound on the polls of one row barrier (each a device-scope load plus a short sleep, about a
// microsecond): every wave leaves the barrier after at most about a second even if a workgroup
// of the row never arrived, so the launch always drains (the row's result is then wrong).
constexpr uint32_t SP_SPIN_LIMIT = 1u << 20;

// Barrier of the workgroups of one row inside one launch, round `round` (1, 2, ..): each wave
// waits until its own global stores and atomics have completed and the workgroup meets; then
// one thread counts the workgroup in. Chunks of rows longer than 32 chunks are counted in eight
// groups (c % 8), so no single word takes every arrival of a long row: the last arrival of a
// group counts the group in, and the last group (or, in shorter rows, the last arrival) sets
// every group's release word; each workgroup polls only its group's. Deadlock-free when every row's workgroups can be resident at once: workgroups are
// dispatched in order, so the lowest unfinished row always has all its workgroups resident and
// finishes.
__device__ __forceinline__ void row_barrier(uint32_t* barw, int c, uint32_t n, uint32_t round) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t g = (uint32_t)c & 7u;
    const uint32_t groups = min(n, 8u);
    const uint32_t in_group = (n + 7u - g) >> 3;
    uint32_t* release = barw + (9 + g) * BAR_STRIDE;
    // rows of at most 32 chunks count every arrival on the row's counter directly (one atomic
    // round trip fewer); longer rows count groups first
    const bool last =
        n <= 32u ? __hip_atomic_fetch_add(barw + 8 * BAR_STRIDE, 1u, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT) + 1u == round * n
                 : (__hip_atomic_fetch_add(barw + g * BAR_STRIDE, 1u, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT) + 1u == round * in_group &&
                    __hip_atomic_fetch_add(barw + 8 * BAR_STRIDE, 1u, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT) + 1u == round * groups);
    if (last) {
      for (uint32_t j = 0; j < groups; ++j)
        __hip_atomic_store(barw + (9 + j) * BAR_STRIDE, round, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    for (uint32_t spin = 0; spin < SP_SPIN_LIMIT; ++spin) {
      if (__hip_atomic_load(release, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= round) break;
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __syncthreads();
}

__device__ __forceinline__ SplitChunk split_chunk(const float* scores, int64_t ld,
                                                  const int32_t* cu_q, const int64_t* cu_k,
                                                  int nseq, int64_t total_k, int k,
                                                  int max_k, int max_chunks) {
  SplitChunk r;
  r.t = blockIdx.x / max_chunks;
  r.c = blockIdx.x - r.t * max_chunks;
  const QueryPos qp = query_pos(cu_q, cu_k, nseq, total_k, r.t);
  // a row is never longer than the batch's longest sequence, which sized the workspace
  const int64_t n = min(min(qp.p + 1, ld), (int64_t)max_k);
  r.ni = (int)max((int64_t)0, n);
  r.dense = n <= k;
  r.srow = scores + (int64_t)r.t * ld;
  r.off = (int)((reinterpret_cast<uintptr_t>(r.srow) >> 2) & 3);
  r.g4 = reinterpret_cast<const f32x4*>(r.srow - r.off);
  r.ng4 = (r.ni + r.off + 3) >> 2;
  r.nchunks = (r.ng4 + SP_CHUNK4 - 1) / SP_CHUNK4;
  return r;
}

// Unit u of this lane is group c*SP_CHUNK4 + wave*SP_SLICE4 + 64*u + lane; its element e is
// position 4*group + e - off. Slots outside the row hold NaN.
__device__ __forceinline__ void split_load(const SplitChunk& r, float (&x)[SP_UNITS][4]) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const float qnan = __uint_as_float(0x7fc00000u);
#pragma unroll
  for (int u = 0; u < SP_UNITS; ++u) {
    const int g = r.c * SP_CHUNK4 + wave * SP_SLICE4 + u * WAVE + lane;
    f32x4 v = {qnan, qnan, qnan, qnan};
    if (g < r.ng4) v = r.g4[g];
#pragma unroll
    for (int e = 0; e < 4; ++e) x[u][e] = v[e];
    if (g == 0 || g == r.ng4 - 1) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int pos = 4 * g + e - r.off;
        if (pos < 0 || pos >= r.ni) x[u][e] = qnan;
      }
    }
  }
}

// Workgroup-wide min and max (NaN ignored). Two barriers.
__device__ __forceinline__ void wg_minmax(float& mn, float& mx, SplitShared& sh) {
  const int wave = threadIdx.x >> 6;
  mn = __uint_as_float(last_lane(wave_incl_scan(__float_as_uint(mn), 0x7f800000u, MinF32())));
  mx = __uint_as_float(last_lane(wave_incl_scan(__float_as_uint(mx), 0xff800000u, MaxF32())));
  if (lane_id() == 0) { sh.red_a[wave] = __float_as_uint(mn); sh.red_b[wave] = __float_as_uint(mx); }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < SP_WAVES; ++w) {
    mn = fminf(mn, __uint_as_float(sh.red_a[w]));
    mx = fmaxf(mx, __uint_as_float(sh.red_b[w]));
  }
  __syncthreads();
}

// Workgroup-wide sums of two counts. Two barriers.
__device__ __forceinline__ void wg_sum2(uint32_t& a, uint32_t& b, SplitShared& sh) {
  const int wave = threadIdx.x >> 6;
  a = last_lane(wave_incl_scan_u32(a));
  b = last_lane(wave_incl_scan_u32(b));
  if (lane_id() == 0) { sh.red_c[wave] = a; sh.red_d[wave] = b; }
  __syncthreads();
  a = 0;
  b = 0;
#pragma unroll
  for (int w = 0; w < SP_WAVES; ++w) { a += sh.red_c[w]; b += sh.red_d[w]; }
  __syncthreads();
}

// This thread's slice (SP_BPT consecutive bins) of a histogram and, optionally, of its bins'
// smallest and largest keys. The split kernels load the slices of the row's global histograms
// right after the sequence lookup, ahead of their chunk's scores, so that the selects run while
// the scores are still arriving.
struct SplitSlice {
  uint32_t h[SP_BPT], mn[SP_BPT], mx[SP_BPT];
};

template <bool COH = false>
__device__ __forceinline__ void split_slice_load(const uint32_t* h, const uint32_t* mn,
                                                 const uint32_t* mx, SplitSlice& sl) {
  const int b = SP_BPT * threadIdx.x;
#pragma unroll
  for (int j = 0; j < SP_BPT; ++j) {
    sl.h[j] = ws_ld<COH>(h + b + j);
    sl.mn[j] = mn ? ws_ld<COH>(mn + b + j) : 0u;
    sl.mx[j] = mx ? ws_ld<COH>(mx + b + j) : 0u;
  }
}

// The row's fine histogram with its bins' extremes, as slices. The workspace holds each bin's
// smallest key complemented (kept with atomicMax), so a cleared row state is all zero.
template <bool COH = false>
__device__ __forceinline__ void split_fine_load(const uint32_t* rw, SplitSlice& sl) {
  const int b = SP_BPT * threadIdx.x;
#pragma unroll
  for (int j = 0; j < SP_BPT; ++j) {
    sl.h[j] = ws_ld<COH>(rw + RW_HIST1 + b + j);
    sl.mn[j] = ~ws_ld<COH>(rw + RW_MIN1 + b + j);
    sl.mx[j] = ws_ld<COH>(rw + RW_MAX1 + b + j);
  }
}

// In a histogram held as per-thread slices (keys counted from the top bin down), finds the bin
// holding the need-th largest key and publishes it with the keys still needed from it, its
// count and its smallest and largest key (as the slices hold them). If the histogram holds
// fewer than `need` keys, sel_count is 0. Three barriers (the first one lets every thread finish
// reading the previous select's results).
__device__ __forceinline__ void split_select(const SplitSlice& sl, uint32_t need,
                                             SplitShared& sh) {
  __syncthreads();
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  uint32_t hv[SP_BPT];
  uint32_t s = 0;
#pragma unroll
  for (int j = 0; j < SP_BPT; ++j) {
    hv[j] = sl.h[j];
    s += hv[j];
  }
  const uint32_t incl = wave_incl_scan_u32(s);
  const uint32_t wave_tot = last_lane(incl);
  if (lane_id() == 0) sh.red_a[wave] = wave_tot;
  if (tid == 0) { sh.sel_bin = 0; sh.sel_need = need; sh.sel_count = 0; sh.sel_min = 0; sh.sel_max = 0; }
  __syncthreads();
  uint32_t above = wave_tot - incl;              // keys in bins above this thread's bins
#pragma unroll
  for (int w = 0; w < SP_WAVES; ++w)
    if (w > wave) above += sh.red_a[w];
#pragma unroll
  for (int j = SP_BPT - 1; j >= 0; --j) {
    if (above < need && above + hv[j] >= need) {
      const int b = SP_BPT * tid + j;
      sh.sel_bin = b;
      sh.sel_need = need - above;
      sh.sel_count = hv[j];
      sh.sel_min = sl.mn[j];
      sh.sel_max = sl.mx[j];
    }
    above += hv[j];
  }
  __syncthreads();
}

// The same on a histogram in memory (global or LDS; mn / mx may be null).
__device__ __forceinline__ void split_select(const uint32_t* h, const uint32_t* mn,
                                             const uint32_t* mx, uint32_t need,
                                             SplitShared& sh) {
  SplitSlice sl;
  split_slice_load(h, mn, mx, sl);
  split_select(sl, need, sh);
}

// Bins of the first two rounds of a row, from its smallest and largest score (every workgroup of
// the row computes the same values).
struct SplitBins {
  int mode;               // 0: one value (or none), 1: linear bins, 2: key bins
  float xmin, xmax;
  float s0, c0;           // linear round 0
  uint32_t lo0;           // key round 0: bin = (key - lo0) >> shift0
  int shift0;
};

// The first SP_THREADS chunk extremes of a row, one per thread (loaded ahead of the scores).
template <bool COH = false>
__device__ __forceinline__ float2 split_minmax_load(const float2* mm, int nchunks) {
  const float inf = __int_as_float(0x7f800000);
  if ((int)threadIdx.x >= nchunks) return make_float2(inf, -inf);
  const uint64_t v = ws_ld64<COH>((const uint64_t*)mm + threadIdx.x);
  return make_float2(__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32)));
}

__device__ __forceinline__ SplitBins split_bins(const float2* mm, float2 first, int nchunks,
                                                SplitShared& sh) {
  float mn = first.x, mx = first.y;
  for (int i = threadIdx.x + SP_THREADS; i < nchunks; i += SP_THREADS) {
    const float2 v = mm[i];
    mn = fminf(mn, v.x);
    mx = fmaxf(mx, v.y);
  }
  wg_minmax(mn, mx, sh);
  SplitBins sb;
  sb.xmin = mn;
  sb.xmax = mx;
  sb.s0 = 0.f;
  sb.c0 = 0.f;
  sb.lo0 = 0;
  sb.shift0 = 0;
  if (!(mn < mx)) {
    sb.mode = 0;
    return sb;
  }
  const float s0 = (float)TK_BINS / (mx - mn);
  if (s0 > 0.f && s0 <= __FLT_MAX__) {
    sb.mode = 1;
    sb.s0 = s0;
    sb.c0 = -mn * s0;
  } else {
    sb.mode = 2;
    sb.lo0 = score_key(mn);
    const uint32_t span = score_key(mx) - sb.lo0;
    int shift = 0;
    while ((span >> shift) >= (uint32_t)TK_BINS) ++shift;
    sb.shift0 = shift;
  }
  return sb;
}

__device__ __forceinline__ uint32_t split_bin0(const SplitBins& sb, float v) {
  if (sb.mode == 1) return lin_bin(v, sb.s0, sb.c0);
  return v == v ? (score_key(v) - sb.lo0) >> sb.shift0 : (uint32_t)TK_BINS;
}

// Fine bins inside round-0 bin `bin0`.
struct SplitBins1 {
  float s1, c1;
  uint32_t base1;
  int shift1;
};

__device__ __forceinline__ SplitBins1 split_bins1(const SplitBins& sb, uint32_t bin0) {
  SplitBins1 b1;
  b1.s1 = 0.f;
  b1.c1 = 0.f;
  b1.base1 = 0;
  b1.shift1 = 0;
  if (sb.mode == 1) {
    float s1 = sb.s0 * (float)TK_BINS;
    float c1 = -(sb.xmin + (float)bin0 / sb.s0) * s1;
    if (!(s1 <= __FLT_MAX__ && c1 <= __FLT_MAX__ && c1 >= -__FLT_MAX__)) { s1 = 0.f; c1 = 0.f; }
    b1.s1 = s1;
    b1.c1 = c1;
  } else {
    b1.base1 = sb.lo0 + (bin0 << sb.shift0);
    b1.shift1 = sb.shift0 > 11 ? sb.shift0 - 11 : 0;
  }
  return b1;
}

__device__ __forceinline__ uint32_t split_bin1(const SplitBins& sb, const SplitBins1& b1, float v) {
  if (sb.mode == 1) return lin_bin(v, b1.s1, b1.c1);
  return (score_key(v) - b1.base1) >> b1.shift1;
}

// The chosen fine bin: keys [lo, hi] of which `need` are taken, `count` keys inside it.
struct SplitChoice {
  uint32_t lo, hi, count, need;
};

// h0, h1: the row's round-0 histogram and its fine histogram with bin extremes, as slices.
__device__ __forceinline__ SplitChoice split_choice(const SplitBins& sb, const SplitSlice& h0,
                                                    const SplitSlice& h1, int k,
                                                    SplitShared& sh) {
  SplitChoice ch;
  if (sb.mode == 0) {                            // one value: take the first k of them
    ch.lo = ch.hi = score_key(sb.xmin);
    ch.count = 0xffffffffu;
    ch.need = (uint32_t)k;
    return ch;
  }
  split_select(h0, (uint32_t)k, sh);
  const uint32_t need1 = sh.sel_need;
  split_select(h1, need1, sh);
  ch.lo = sh.sel_min;
  ch.hi = sh.sel_max;
  ch.count = sh.sel_count;
  ch.need = sh.sel_need;
  return ch;
}

__global__ __launch_bounds__(SP_THREADS) void topk_split_prep(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ cu_q,
    const int64_t* __restrict__ cu_k, int nseq, int64_t total_k, int k, SplitWs ws) {
  __shared__ SplitShared sh;
  const SplitChunk r = split_chunk(scores, ld, cu_q, cu_k, nseq, total_k, k, ws.max_k, ws.max_chunks);
  if (r.dense || r.c >= r.nchunks) return;
  float x[SP_UNITS][4];
  split_load(r, x);
  uint32_t* rw = ws.rows + (int64_t)r.t * RW_WORDS;
  for (int i = r.c * SP_THREADS + threadIdx.x; i < RW_WORDS; i += r.nchunks * SP_THREADS)
    rw[i] = 0u;
  float mn = __int_as_float(0x7f800000), mx = -mn;
#pragma unroll
  for (int u = 0; u < SP_UNITS; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      mn = fminf(mn, x[u][e]);
      mx = fmaxf(mx, x[u][e]);
    }
  wg_minmax(mn, mx, sh);
  if (threadIdx.x == 0) ws.minmax[(int64_t)r.t * ws.max_chunks + r.c] = make_float2(mn, mx);
}

__global__ __launch_bounds__(SP_THREADS) void topk_split_hist0(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ cu_q,
    const int64_t* __restrict__ cu_k, int nseq, int64_t total_k, int k, SplitWs ws) {
  __shared__ SplitShared sh;
  const SplitChunk r = split_chunk(scores, ld, cu_q, cu_k, nseq, total_k, k, ws.max_k, ws.max_chunks);
  if (r.dense || r.c >= r.nchunks) return;
  const float2* mm = ws.minmax + (int64_t)r.t * ws.max_chunks;
  const float2 mm0 = split_minmax_load(mm, r.nchunks);
  float x[SP_UNITS][4];
  split_load(r, x);
  for (int i = threadIdx.x; i < TK_BINS; i += SP_THREADS) sh.hist[i] = 0;
  const SplitBins sb = split_bins(mm, mm0, r.nchunks, sh);
  if (sb.mode == 0) return;
#pragma unroll
  for (int u = 0; u < SP_UNITS; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t b = split_bin0(sb, x[u][e]);
      if (b < (uint32_t)TK_BINS) atomicAdd(&sh.hist[b], 1u);
    }
  __syncthreads();
  uint32_t* hg = ws.rows + (int64_t)r.t * RW_WORDS + RW_HIST0;
  for (int i = threadIdx.x; i < TK_BINS; i += SP_THREADS)
    if (sh.hist[i]) atomicAdd(&hg[i], sh.hist[i]);
}

__global__ __launch_bounds__(SP_THREADS) void topk_split_hist1(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ cu_q,
    const int64_t* __restrict__ cu_k, int nseq, int64_t total_k, int k, SplitWs ws) {
  __shared__ SplitShared sh;
  const SplitChunk r = split_chunk(scores, ld, cu_q, cu_k, nseq, total_k, k, ws.max_k, ws.max_chunks);
  if (r.dense || r.c >= r.nchunks) return;
  uint32_t* rw = ws.rows + (int64_t)r.t * RW_WORDS;
  const float2* mm = ws.minmax + (int64_t)r.t * ws.max_chunks;
  const float2 mm0 = split_minmax_load(mm, r.nchunks);
  SplitSlice h0;
  split_slice_load(rw + RW_HIST0, nullptr, nullptr, h0);
  float x[SP_UNITS][4];
  split_load(r, x);
  for (int i = threadIdx.x; i < TK_BINS; i += SP_THREADS) {
    sh.hist[i] = 0;
    sh.bmin[i] = 0xffffffffu;
    sh.bmax[i] = 0u;
  }
  const SplitBins sb = split_bins(mm, mm0, r.nchunks, sh);
  if (sb.mode == 0) return;
  split_select(h0, (uint32_t)k, sh);
  const uint32_t bin0 = sh.sel_bin;
  const SplitBins1 b1 = split_bins1(sb, bin0);
#pragma unroll
  for (int u = 0; u < SP_UNITS; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float v = x[u][e];
      if (split_bin0(sb, v) == bin0) {
        const uint32_t b = split_bin1(sb, b1, v);
        const uint32_t kk = score_key(v);
        atomicAdd(&sh.hist[b], 1u);
        atomicMin(&sh.bmin[b], kk);
        atomicMax(&sh.bmax[b], kk);
      }
    }
  __syncthreads();
  for (int i = threadIdx.x; i < TK_BINS; i += SP_THREADS) {
    const uint32_t h = sh.hist[i];
    if (h) {
      atomicAdd(&rw[RW_HIST1 + i], h);
      atomicMax(&rw[RW_MIN1 + i], ~sh.bmin[i]);
      atomicMax(&rw[RW_MAX1 + i], sh.bmax[i]);
    }
  }
}

// The scores above the chosen fine bin and inside it, per chunk (published in ws.counts); when
// the chosen bin is neither taken whole nor one value, this chunk's positions inside it are
// appended to the row's candidate list.
template <bool COH>
__device__ __forceinline__ void split_count_body(const SplitChunk& r,
                                                 const float (&x)[SP_UNITS][4],
                                                 const SplitChoice& ch, const SplitWs& ws,
                                                 uint32_t* rw, SplitShared& sh) {
  const float vlo = key_value(ch.lo), vhi = key_value(ch.hi);
  uint32_t above = 0, inside = 0;
#pragma unroll
  for (int u = 0; u < SP_UNITS; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float v = x[u][e];
      above += v > vhi;
      inside += v >= vlo && v <= vhi;
    }
  const uint32_t mine = inside;
  wg_sum2(above, inside, sh);
  if (threadIdx.x == 0)
    ws_st64<COH>((uint64_t*)(ws.counts + (int64_t)r.t * ws.max_chunks + r.c),
                 (uint64_t)above | ((uint64_t)inside << 32));
  if (ch.count == ch.need || ch.lo == ch.hi || inside == 0) return;
  // unresolved: append this chunk's positions inside [lo, hi] to the row's candidate list
  const int wave = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_scan_u32(mine);
  if (lane_id() == WAVE - 1) sh.red_a[wave] = incl;
  if (threadIdx.x == 0) sh.bcast = atomicAdd(&rw[RW_CAND_N], inside);
  __syncthreads();
  uint32_t slot = sh.bcast + incl - mine;
  for (int w = 0; w < wave; ++w) slot += sh.red_a[w];
  uint32_t* cand = ws.cand + (int64_t)r.t * ws.cand_cap;
  const int g0 = r.c * SP_CHUNK4 + wave * SP_SLICE4 + lane_id();
#pragma unroll
  for (int u = 0; u < SP_UNITS; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float v = x[u][e];
      if (v >= vlo && v <= vhi) {
        if (slot < ws.cand_cap) {
          ws_st<COH>(cand + slot, (uint32_t)(4 * (g0 + u * WAVE) + e - r.off));
          ws_st<COH>(ws.candk + (int64_t)r.t * ws.cand_cap + slot, score_key(v));
        }
        ++slot;
      }
    }
}

__global__ __launch_bounds__(SP_THREADS) void topk_split_count(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ cu_q,
    const int64_t* __restrict__ cu_k, int nseq, int64_t total_k, int k, SplitWs ws) {
  __shared__ SplitShared sh;
  const SplitChunk r = split_chunk(scores, ld, cu_q, cu_k, nseq, total_k, k, ws.max_k, ws.max_chunks);
  if (r.dense || r.c >= r.nchunks) return;
  uint32_t* rw = ws.rows + (int64_t)r.t * RW_WORDS;
  const float2* mm = ws.minmax + (int64_t)r.t * ws.max_chunks;
  const float2 mm0 = split_minmax_load(mm, r.nchunks);
  SplitSlice h0, h1;
  split_slice_load(rw + RW_HIST0, nullptr, nullptr, h0);
  split_fine_load(rw, h1);
  float x[SP_UNITS][4];
  split_load(r, x);
  const SplitBins sb = split_bins(mm, mm0, r.nchunks, sh);
  const SplitChoice ch = split_choice(sb, h0, h1, k, sh);
  split_count_body<false>(r, x, ch, ws, rw, sh);
}

// The row's candidate list as the compaction reads it: its length and the first SP_CREG *
// SP_THREADS entries (position and key) in registers, loaded in one round with the chunk counts
// (slots past the list hold stale values and are not used).
constexpr int SP_CREG = 4;
struct SplitCands {
  uint32_t n;
  uint32_t pos[SP_CREG], key[SP_CREG];
};

template <bool COH>
__device__ __forceinline__ void split_cands_load(const SplitWs& ws, const uint32_t* rw, int t,
                                                 SplitCands& cd) {
  const uint32_t* cand = ws.cand + (int64_t)t * ws.cand_cap;
  const uint32_t* candk = ws.candk + (int64_t)t * ws.cand_cap;
  cd.n = (uint32_t)min((int64_t)ws_ld<COH>(rw + RW_CAND_N), ws.cand_cap);
#pragma unroll
  for (int j = 0; j < SP_CREG; ++j) {
    const int64_t i = min((int64_t)(threadIdx.x + j * SP_THREADS), ws.cand_cap - 1);
    cd.pos[j] = ws_ld<COH>(cand + i);
    cd.key[j] = ws_ld<COH>(candk + i);
  }
}

// Threshold among the candidates (keys [lo, hi], `count` of them, `need` to take), in rounds of
// 2048 key bins of a power-of-two width: the score T and how many scores equal to T are taken
// (all of them when thr_need is 0xffffffff).
template <bool COH>
__device__ __forceinline__ void split_resolve_candidates(const SplitCands& cd,
                                                         const uint32_t* candk,
                                                         SplitChoice ch, float& thr,
                                                         uint32_t& thr_need, SplitShared& sh) {
  uint32_t lo = ch.lo, hi = ch.hi, count = ch.count, need = ch.need;
  for (;;) {
    if (count == need) { thr = key_value(lo); thr_need = 0xffffffffu; return; }
    if (lo == hi || count == 0) { thr = key_value(lo); thr_need = need; return; }
    const uint32_t span = hi - lo;
    int shift = 0;
    while ((span >> shift) >= (uint32_t)TK_BINS) ++shift;
    for (int i = threadIdx.x; i < TK_BINS; i += SP_THREADS) {
      sh.hist[i] = 0;
      sh.bmin[i] = 0xffffffffu;
      sh.bmax[i] = 0u;
    }
    __syncthreads();
    auto add = [&](uint32_t kk) {
      if (kk >= lo && kk <= hi) {
        const uint32_t b = (kk - lo) >> shift;
        atomicAdd(&sh.hist[b], 1u);
        atomicMin(&sh.bmin[b], kk);
        atomicMax(&sh.bmax[b], kk);
      }
    };
#pragma unroll
    for (int j = 0; j < SP_CREG; ++j)
      if (threadIdx.x + j * SP_THREADS < cd.n) add(cd.key[j]);
    for (uint32_t i = threadIdx.x + SP_CREG * SP_THREADS; i < cd.n; i += SP_THREADS)
      add(ws_ld<COH>(candk + i));
    __syncthreads();
    split_select(sh.hist, sh.bmin, sh.bmax, need, sh);
    count = sh.sel_count;
    need = sh.sel_need;
    lo = sh.sel_min;
    hi = sh.sel_max;
    __syncthreads();                             // hist is cleared by the next round
  }
}

// Resolves the threshold and writes this chunk's selected positions in index order. above_b /
// inside_b: this thread's share of the counts of the chunks before this one.
template <bool COH>
__device__ __forceinline__ void split_compact_body(const SplitChunk& r,
                                                   const float (&x)[SP_UNITS][4],
                                                   const SplitChoice& ch, uint32_t above_b,
                                                   uint32_t inside_b, const SplitCands& cd,
                                                   const SplitWs& ws, int k, int32_t* orow,
                                                   SplitShared& sh) {
  wg_sum2(above_b, inside_b, sh);
  float thr;
  uint32_t thr_need, gt_before, eq_before;
  if (ch.count == ch.need) {                     // the whole fine bin is taken
    thr = key_value(ch.lo);
    thr_need = 0xffffffffu;
    gt_before = above_b + inside_b;
    eq_before = 0;
  } else if (ch.lo == ch.hi) {                   // one value: the first `need` of it are taken
    thr = key_value(ch.lo);
    thr_need = ch.need;
    gt_before = above_b;
    eq_before = inside_b;
  } else {
    const uint32_t* cand = ws.cand + (int64_t)r.t * ws.cand_cap;
    const uint32_t* candk = ws.candk + (int64_t)r.t * ws.cand_cap;
    split_resolve_candidates<COH>(cd, candk, ch, thr, thr_need, sh);
    // candidates of the chunks before this one above / equal to the threshold (in key space)
    const int first_pos = 4 * r.c * SP_CHUNK4 - r.off;
    const uint32_t tk = score_key(thr);
    uint32_t gt = 0, eq = 0;
    auto tally = [&](uint32_t pos, uint32_t kk) {
      if ((int)pos < first_pos) {
        gt += kk > tk;
        eq += kk == tk;
      }
    };
#pragma unroll
    for (int j = 0; j < SP_CREG; ++j)
      if (threadIdx.x + j * SP_THREADS < cd.n) tally(cd.pos[j], cd.key[j]);
    for (uint32_t i = threadIdx.x + SP_CREG * SP_THREADS; i < cd.n; i += SP_THREADS)
      tally(ws_ld<COH>(cand + i), ws_ld<COH>(candk + i));
    wg_sum2(gt, eq, sh);
    gt_before = above_b + gt;
    eq_before = eq;
  }
  // compaction of this chunk in index order
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int u = 0; u < SP_UNITS; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      gt += (uint32_t)__popcll(__ballot(x[u][e] > thr));
      eq += (uint32_t)__popcll(__ballot(x[u][e] == thr));
    }
  if (lane == 0) { sh.red_c[wave] = gt; sh.red_d[wave] = eq; }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < SP_WAVES; ++w)
    if (w < wave) { gt_before += sh.red_c[w]; eq_before += sh.red_d[w]; }
  uint32_t eqc = eq_before;
  uint32_t base = gt_before + min(eq_before, thr_need);
  const int g0 = r.c * SP_CHUNK4 + wave * SP_SLICE4 + lane;
#pragma unroll
  for (int u = 0; u < SP_UNITS; ++u) {
    uint64_t tm[4];
    uint64_t eq_any = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tm[e] = __ballot(x[u][e] > thr);
      eq_any |= __ballot(x[u][e] == thr);
    }
    if (eq_any) {
      uint64_t qm[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) qm[e] = __ballot(x[u][e] == thr);
      uint32_t rank = eqc;
#pragma unroll
      for (int e = 0; e < 4; ++e) rank += lanes_below(qm[e]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool is_eq = x[u][e] == thr;
        tm[e] |= __ballot(is_eq && rank < thr_need);
        rank += is_eq;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) eqc += (uint32_t)__popcll(qm[e]);
    }
    uint32_t slot = base;
#pragma unroll
    for (int e = 0; e < 4; ++e) slot += lanes_below(tm[e]);
    const int p0 = 4 * (g0 + u * WAVE) - r.off;
    const uint64_t lane_bit = 1ull << lane;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (tm[e] & lane_bit) {
        if (slot < (uint32_t)k) orow[slot] = p0 + e;
        ++slot;
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) base += (uint32_t)__popcll(tm[e]);
  }
}

__global__ __launch_bounds__(SP_THREADS) void topk_split_compact(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ cu_q,
    const int64_t* __restrict__ cu_k, int nseq, int64_t total_k, int k, SplitWs ws,
    int32_t* __restrict__ out) {
  __shared__ SplitShared sh;
  const SplitChunk r = split_chunk(scores, ld, cu_q, cu_k, nseq, total_k, k, ws.max_k, ws.max_chunks);
  int32_t* orow = out + (int64_t)r.t * k;
  if (r.dense) {
    if (r.c == 0)
      for (int i = threadIdx.x; i < k; i += SP_THREADS) orow[i] = i < r.ni ? i : -1;
    return;
  }
  if (r.c >= r.nchunks) return;
  const uint32_t* rw = ws.rows + (int64_t)r.t * RW_WORDS;
  const float2* mm = ws.minmax + (int64_t)r.t * ws.max_chunks;
  const float2 mm0 = split_minmax_load(mm, r.nchunks);
  SplitSlice h0, h1;
  split_slice_load(rw + RW_HIST0, nullptr, nullptr, h0);
  split_fine_load(rw, h1);
  SplitCands cd;
  split_cands_load<false>(ws, rw, r.t, cd);
  // counts of the chunks before this one
  uint32_t above_b = 0, inside_b = 0;
  const uint2* cnt = ws.counts + (int64_t)r.t * ws.max_chunks;
  for (int i = threadIdx.x; i < r.c; i += SP_THREADS) {
    const uint2 v = cnt[i];
    above_b += v.x;
    inside_b += v.y;
  }
  float x[SP_UNITS][4];
  split_load(r, x);
  const SplitBins sb = split_bins(mm, mm0, r.nchunks, sh);
  const SplitChoice ch = split_choice(sb, h0, h1, k, sh);
  split_compact_body<false>(r, x, ch, above_b, inside_b, cd, ws, k, orow, sh);
}

// Zero-fills the row state of the one-launch path (when no earlier launch of the step did).
__global__ __launch_bounds__(256) void topk_split_clear(uint32_t* __restrict__ rows, int64_t words) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < words) rows[i] = 0u;
}

// The split path in one launch: the workgroups of a row meet at three row barriers instead of
// launch boundaries, and each loads its chunk once. Round 0 bins the order-preserving key's top
// bits instead of the range between the row's extremes, which saves the extremes' pass. Every value another
// workgroup of the row produced is read through device-scope atomics (ws_ld), and every value
// this one publishes is written the same way or with global atomics. Requires the row state
// zero-filled (topk_split_clear, or an earlier launch of the step) and at most SP_THREADS chunks
// per row.
__global__ __launch_bounds__(SP_THREADS) void topk_split_fused(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ cu_q,
    const int64_t* __restrict__ cu_k, int nseq, int64_t total_k, int k, SplitWs ws,
    int32_t* __restrict__ out) {
  __shared__ SplitShared sh;
  const SplitChunk r = split_chunk(scores, ld, cu_q, cu_k, nseq, total_k, k, ws.max_k, ws.max_chunks);
  int32_t* orow = out + (int64_t)r.t * k;
  if (r.dense) {
    if (r.c == 0)
      for (int i = threadIdx.x; i < k; i += SP_THREADS) orow[i] = i < r.ni ? i : -1;
    return;
  }
  if (r.c >= r.nchunks) return;
  uint32_t* rw = ws.rows + (int64_t)r.t * RW_WORDS;
  uint32_t* bar = rw + RW_BAR;
  const uint32_t n = (uint32_t)r.nchunks;
  float x[SP_UNITS][4];
  split_load(r, x);

  // 1. round-0 histogram of the row: 2048 bins of the order-preserving key's top 11 bits
  // (no pass over the row's extremes first; the fine round splits the chosen bin by the next 11)
  SplitBins sb;
  sb.mode = 2;
  sb.xmin = sb.xmax = 0.f;
  sb.s0 = sb.c0 = 0.f;
  sb.lo0 = 0;
  sb.shift0 = 21;
  for (int i = threadIdx.x; i < TK_BINS; i += SP_THREADS) sh.hist[i] = 0;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < SP_UNITS; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t b = split_bin0(sb, x[u][e]);
      if (b < (uint32_t)TK_BINS) atomicAdd(&sh.hist[b], 1u);
    }
  __syncthreads();
  for (int i = threadIdx.x; i < TK_BINS; i += SP_THREADS)
    if (sh.hist[i]) atomicAdd(&rw[RW_HIST0 + i], sh.hist[i]);
  row_barrier(bar, r.c, n, 1);

  // 2. the bin holding the k-th largest score, split into 2048 fine bins of 2^10 keys (counts
  // only: a fine bin's key range is known, and an unresolved one goes through the candidates)
  SplitSlice h0;
  split_slice_load<true>(rw + RW_HIST0, nullptr, nullptr, h0);
  for (int i = threadIdx.x; i < TK_BINS; i += SP_THREADS) sh.hist[i] = 0;
  split_select(h0, (uint32_t)k, sh);            // (its first barrier orders the clear)
  const uint32_t bin0 = sh.sel_bin;
  const SplitBins1 b1 = split_bins1(sb, bin0);
#pragma unroll
  for (int u = 0; u < SP_UNITS; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float v = x[u][e];
      if (split_bin0(sb, v) == bin0) atomicAdd(&sh.hist[split_bin1(sb, b1, v)], 1u);
    }
  __syncthreads();
  for (int i = threadIdx.x; i < TK_BINS; i += SP_THREADS)
    if (sh.hist[i]) atomicAdd(&rw[RW_HIST1 + i], sh.hist[i]);
  row_barrier(bar, r.c, n, 2);

  // 3. counts above and inside the chosen fine bin; candidates when it is unresolved
  SplitSlice h1;
  {
    const int bb = SP_BPT * threadIdx.x;
#pragma unroll
    for (int j = 0; j < SP_BPT; ++j) {
      // the bin's keys, clamped to those of finite or infinite scores (the keys outside
      // [key(-inf), key(+inf)] are NaN patterns, which would fail every range comparison)
      const uint32_t lo = b1.base1 + ((uint32_t)(bb + j) << b1.shift1);
      h1.h[j] = ws_ld<true>(rw + RW_HIST1 + bb + j);
      h1.mn[j] = max(lo, 0x007fffffu);
      h1.mx[j] = min(lo + ((1u << b1.shift1) - 1u), 0xff800000u);
    }
  }
  const SplitChoice ch = split_choice(sb, h0, h1, k, sh);
  split_count_body<true>(r, x, ch, ws, rw, sh);
  row_barrier(bar, r.c, n, 3);

  // 4. compaction: the earlier chunks' counts and the candidate list in one round of loads
  SplitCands cd;
  split_cands_load<true>(ws, rw, r.t, cd);
  uint32_t above_b = 0, inside_b = 0;
  const uint64_t* cnt = (const uint64_t*)(ws.counts + (int64_t)r.t * ws.max_chunks);
  for (int i = threadIdx.x; i < r.c; i += SP_THREADS) {
    const uint64_t v = ws_ld64<true>(cnt + i);
    above_b += (uint32_t)v;
    inside_b += (uint32_t)(v >> 32);
  }
  split_compact_body<true>(r, x, ch, above_b, inside_b, cd, ws, k, orow, sh);
}

// Layout of the split workspace for this batch; rows.. cand are null when ws is null.
struct SplitLayout {
  int max_chunks;
  int64_t cand_cap;
  size_t rows_off, minmax_off, counts_off, cand_off, candk_off, bytes;
};

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

SplitLayout split_layout(const Batch& b) {
  SplitLayout L;
  const int64_t groups = ((int64_t)b.max_k + 3) / 4 + 1;
  L.max_chunks = (int)((groups + SP_CHUNK4 - 1) / SP_CHUNK4);
  L.cand_cap = ((int64_t)b.max_k + 63) & ~(int64_t)63;
  const size_t T = (size_t)b.total_q;
  L.rows_off = 0;
  L.minmax_off = align256(T * RW_WORDS * sizeof(uint32_t));
  L.counts_off = L.minmax_off + align256(T * L.max_chunks * sizeof(float2));
  L.cand_off = L.counts_off + align256(T * L.max_chunks * sizeof(uint2));
  L.candk_off = L.cand_off + align256(T * (size_t)L.cand_cap * sizeof(uint32_t));
  L.bytes = L.candk_off + align256(T * (size_t)L.cand_cap * sizeof(uint32_t));
  return L;
}

// Split rows when the batch has too few rows to fill the chip with one workgroup per row and
// the rows are longer than one register-resident chunk of the single-workgroup kernel.
bool use_split(const Batch& b, int k) {
  return b.max_k > 4 * TK_THREADS * 8 && b.max_k > k && b.total_q <= 64;
}

// Workgroups of topk_split_fused the current device holds at once (its compute units times the
// kernel's occupancy per compute unit), found once per device: a row's barriers need all of the
// row's workgroups resident, which a partitioned device with fewer compute units may not allow.
int64_t fused_resident_capacity() {
  static std::mutex mu;
  static std::map<int, int64_t> cap;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cap.find(dev);
  if (it != cap.end()) return it->second;
  int cus = 0, per_cu = 0;
  int64_t c = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, topk_split_fused, SP_THREADS, 0) ==
          hipSuccess)
    c = (int64_t)cus * per_cu;
  cap[dev] = c;
  return c;
}

// The one-launch path: rows of at most 256 chunks whose workgroups the device holds at once.
bool one_launch_fits(int max_chunks) {
  return max_chunks <= SP_THREADS && (int64_t)max_chunks <= fused_resident_capacity();
}

hipError_t launch_split(const Batch& b, const float* scores, int64_t ld, int k, int32_t* indices,
                        void* workspace, bool state_zeroed, hipStream_t stream) {
  const SplitLayout L = split_layout(b);
  char* base = (char*)workspace;
  SplitWs ws;
  ws.rows = (uint32_t*)(base + L.rows_off);
  ws.minmax = (float2*)(base + L.minmax_off);
  ws.counts = (uint2*)(base + L.counts_off);
  ws.cand = (uint32_t*)(base + L.cand_off);
  ws.candk = (uint32_t*)(base + L.candk_off);
  ws.max_chunks = L.max_chunks;
  ws.max_k = b.max_k;
  ws.cand_cap = L.cand_cap;
  const unsigned grid = (unsigned)((int64_t)b.total_q * L.max_chunks);
  if (one_launch_fits(L.max_chunks)) {
    // one launch once the row state is zero: at most 64 rows of at most 256 chunks are 16384
    // workgroups of 256 threads, of which one row's (at most 256) are always resident
    const int64_t words = (int64_t)b.total_q * RW_WORDS;
    if (!state_zeroed)
      topk_split_clear<<<(unsigned)((words + 255) / 256), 256, 0, stream>>>(ws.rows, words);
    topk_split_fused<<<grid, SP_THREADS, 0, stream>>>(scores, ld, b.cu_q, b.cu_k, b.nseq,
                                                      b.total_k, k, ws, indices);
    return hipGetLastError();
  }
  topk_split_prep<<<grid, SP_THREADS, 0, stream>>>(scores, ld, b.cu_q, b.cu_k, b.nseq, b.total_k,
                                                   k, ws);
  topk_split_hist0<<<grid, SP_THREADS, 0, stream>>>(scores, ld, b.cu_q, b.cu_k, b.nseq,
                                                    b.total_k, k, ws);
  topk_split_hist1<<<grid, SP_THREADS, 0, stream>>>(scores, ld, b.cu_q, b.cu_k, b.nseq,
                                                    b.total_k, k, ws);
  topk_split_count<<<grid, SP_THREADS, 0, stream>>>(scores, ld, b.cu_q, b.cu_k, b.nseq,
                                                    b.total_k, k, ws);
  topk_split_compact<<<grid, SP_THREADS, 0, stream>>>(scores, ld, b.cu_q, b.cu_k, b.nseq,
                                                      b.total_k, k, ws, indices);
  return hipGetLastError();
}

template <int UNITS, int MODE, int THREADS = TK_THREADS>
hipError_t launch_rows(const Batch& b, const float* scores, int64_t ld, int k, int32_t* indices,
                       hipStream_t stream) {
  topk_rows<THREADS, UNITS, MODE><<<b.total_q, THREADS, 0, stream>>>(
      scores, ld, b.cu_q, b.cu_k, b.nseq, b.total_q, b.total_k, k, indices);
  return hipGetLastError();
}

}  // namespace

size_t topk_workspace_bytes(const Batch& b, int k) {
  return use_split(b, k) ? split_layout(b).bytes : 0;
}

int64_t topk_state_words(const Batch& b, int k) {
  if (!use_split(b, k)) return 0;
  const SplitLayout L = split_layout(b);
  return one_launch_fits(L.max_chunks) ? (int64_t)b.total_q * RW_WORDS : 0;
}

hipError_t launch_topk(const Batch& b, const float* scores, int64_t ld, int k, int32_t* indices,
                       void* workspace, hipStream_t stream, bool state_zeroed) {
  if (use_split(b, k))
    return launch_split(b, scores, ld, k, indices, workspace, state_zeroed, stream);
  // Registers per thread sized for the longest visible row (16-byte groups, plus one when rows
  // do not all start on a 16-byte boundary); rows longer than 32K keys are processed in chunks.
  const int64_t longest = std::min<int64_t>(b.max_k, ld);
  const bool aligned = (reinterpret_cast<uintptr_t>(scores) & 15) == 0 && ld % 4 == 0;
  const int64_t groups = (longest + 3) / 4 + (aligned ? 0 : 1);
  if (groups <= 1 * TK_THREADS) return launch_rows<1, 0>(b, scores, ld, k, indices, stream);
  if (groups <= 2 * TK_THREADS) return launch_rows<2, 0>(b, scores, ld, k, indices, stream);
  if (groups <= 4 * TK_THREADS) return launch_rows<4, 0>(b, scores, ld, k, indices, stream);
  if (groups <= 8 * TK_THREADS) return launch_rows<8, 0>(b, scores, ld, k, indices, stream);
  // Streamed rows: with enough rows to give every CU two, 512-thread workgroups of half the
  // chunk let two of them share a CU, so one's barriers and memory waits overlap the other's work.
  if (k <= TK_OBUF && b.total_q >= 512) return launch_rows<8, 1, 512>(b, scores, ld, k, indices, stream);
  if (k <= TK_OBUF) return launch_rows<8, 1>(b, scores, ld, k, indices, stream);
  return launch_rows<8, 2>(b, scores, ld, k, indices, stream);
}

}  // namespace dsa

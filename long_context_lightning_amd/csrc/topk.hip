// Causal per-query top-k ("How GLM5.3 Sparse Attention Affects HBM Memory Usage", How it works /
// Model: top-k 2048, dense below 2K visible tokens, one selection shared by all heads).
//
// Selection rule: the k largest scores among positions 0..p, scores compared as reals
// (-0.0 == +0.0), an equal score going to the lower position; output ascending, -1 padded.
// Scores are finite or infinite; a NaN score is never selected.
//
// One workgroup of 1024 threads per query row; the scores stay in registers:
//   * the row is cut into chunks of UNITS*4096 positions (UNITS <= 8); inside a chunk, wave w
//     owns a contiguous slice and lane l of it holds UNITS 16-byte groups, (u*64 + l) within it.
//     A row of at most one chunk is read from memory once; longer rows re-read their chunks on
//     every pass. Slots outside the row hold NaN, which no comparison or bin counts;
//   * round 0 histograms every score into 2048 bins linear in the value between the row's
//     smallest and largest score; round 1 splits the bin holding the k-th largest score into
//     2048 finer linear bins; later rounds split the chosen bin in the space of order-preserving
//     32-bit keys into bins of a power-of-two width (at most three such rounds reach one key).
//     Bin indices are monotone functions of the score (a rounded fused multiply-add, clamped
//     and truncated), so every bin is a contiguous range of scores. From round 1 on each bin
//     also records its smallest and largest key. The bin holding the k-th largest score is found
//     with DPP wave prefix sums and one exchange of wave totals. The select ends when the scores
//     still needed from the chosen bin are all of its scores (everything at or above its
//     smallest score is taken) or when the bin holds a single value. The result is a threshold
//     score T and a count `need`: a position is selected if its score is above T, or equal to T
//     and among the first `need` such positions;
//   * compaction in index order: per chunk, the per-wave counts (ballot popcounts) are
//     exchanged once, which gives each wave its first output slot and the number of scores
//     equal to T before its slice; inside the wave, each step of 256 positions ranks its taken
//     positions with lane-mask counts.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace dsa {
namespace {

constexpr int TK_THREADS = 1024;
constexpr int TK_WAVES = TK_THREADS / WAVE;
constexpr int TK_BINS = 2048;
constexpr int TK_HIST = TK_BINS + 64;          // bin TK_BINS collects NaN (never selected)

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
};

// Finds, in histogram h (bins 2*tid and 2*tid+1 per thread, keys counted from the top bin
// down), the bin holding the need-th largest key, and publishes it with the keys still needed
// from it, its count and its smallest and largest key. Two barriers; all threads must call.
__device__ __forceinline__ void select_bin(const uint32_t* h, const uint32_t* bmin,
                                           const uint32_t* bmax, uint32_t need,
                                           TopkShared& sh) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const uint32_t h0 = h[2 * tid], h1 = h[2 * tid + 1];
  const uint32_t incl = wave_incl_scan_u32(h0 + h1);
  const uint32_t wave_tot = last_lane(incl);
  if (lane_id() == 0) sh.red_a[wave] = wave_tot;
  __syncthreads();
  uint32_t above = wave_tot - incl;            // keys in bins above this thread's two bins
#pragma unroll
  for (int w = 0; w < TK_WAVES; ++w)
    if (w > wave) above += sh.red_a[w];
  int b = -1;
  if (above < need && above + h1 >= need) {
    b = 2 * tid + 1;
    sh.sel_need = need - above;
    sh.sel_count = h1;
  } else if (above + h1 < need && above + h1 + h0 >= need) {
    b = 2 * tid;
    sh.sel_need = need - above - h1;
    sh.sel_count = h0;
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

template <int UNITS>
__global__ __launch_bounds__(TK_THREADS) void topk_rows(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ cu_q,
    const int64_t* __restrict__ cu_k, int nseq, int total_q, int64_t total_k, int k,
    int32_t* __restrict__ out) {
  __shared__ TopkShared sh;
  constexpr int SLICE4 = UNITS * WAVE;           // 16-byte groups per wave and chunk
  constexpr int CHUNK4 = UNITS * TK_THREADS;     // 16-byte groups per chunk
  constexpr uint32_t ALL = 0xffffffffu;

  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  const QueryPos qp = query_pos(cu_q, cu_k, nseq, total_k, t);
  const int64_t n = min(qp.p + 1, ld);           // visible positions 0..n-1 (0 if invalid)
  int32_t* orow = out + (int64_t)t * k;
  if (n <= k) {                                  // dense path: everything visible is selected
    for (int i = tid; i < k; i += TK_THREADS) orow[i] = i < n ? i : -1;
    return;
  }
  const float* srow = scores + (int64_t)t * ld;
  // The row is read in aligned 16-byte groups; `off` floats of the first group precede it.
  // Positions fit in 32 bits (they are stored as int32).
  const int off = (int)((reinterpret_cast<uintptr_t>(srow) >> 2) & 3);
  const f32x4* g4 = reinterpret_cast<const f32x4*>(srow - off);
  const int ni = (int)n;
  const int ng4 = (ni + off + 3) >> 2;
  const int nchunks = (ng4 + CHUNK4 - 1) / CHUNK4;
  const int lane_g = wave * SLICE4 + lane;       // group of unit 0 in chunk 0
  const float qnan = __uint_as_float(0x7fc00000u);

  float x[UNITS][4];
  // Unit u of this lane in chunk c is group c*CHUNK4 + lane_g + 64*u; its element e is
  // position 4*group + e - off.
  auto load_chunk = [&](int c) {
#pragma unroll
    for (int u = 0; u < UNITS; ++u) {
      const int g = c * CHUNK4 + lane_g + u * WAVE;
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
  // f(c) for every chunk with x[][] holding that chunk
  auto for_chunks = [&](auto&& f) {
    if (nchunks == 1) {
      f(0);
    } else {
      for (int c = 0; c < nchunks; ++c) {
        load_chunk(c);
        f(c);
      }
    }
  };
  if (nchunks == 1) load_chunk(0);

  for (int i = tid; i < TK_HIST; i += TK_THREADS) {
    sh.hist[0][i] = 0;
    sh.hist[1][i] = 0;
  }
  for (int i = tid; i < TK_BINS; i += TK_THREADS) {
    sh.bmin[0][i] = ALL;
    sh.bmin[1][i] = ALL;
    sh.bmax[0][i] = 0u;
    sh.bmax[1][i] = 0u;
  }

  // value range of the row (fminf / fmaxf skip NaN)
  float xmin = __int_as_float(0x7f800000), xmax = -xmin;
  for_chunks([&](int) {
#pragma unroll
    for (int u = 0; u < UNITS; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xmin = fminf(xmin, x[u][e]);
        xmax = fmaxf(xmax, x[u][e]);
      }
  });
  xmin = __uint_as_float(last_lane(wave_incl_scan(__float_as_uint(xmin), 0x7f800000u, MinF32())));
  xmax = __uint_as_float(last_lane(wave_incl_scan(__float_as_uint(xmax), 0xff800000u, MaxF32())));
  if (lane == 0) { sh.red_a[wave] = __float_as_uint(xmin); sh.red_b[wave] = __float_as_uint(xmax); }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < TK_WAVES; ++w) {
    xmin = fminf(xmin, __uint_as_float(sh.red_a[w]));
    xmax = fmaxf(xmax, __uint_as_float(sh.red_b[w]));
  }

  // radix select
  uint32_t need = (uint32_t)k;                   // scores to take from the current range
  float thr = xmin;
  uint32_t thr_need = need;
  do {
    if (!(xmin < xmax)) break;                   // a single value: take k of them
    // round 0: linear bins over [xmin, xmax]
    const float s0 = (float)TK_BINS / (xmax - xmin);
    uint32_t lo, hi, count;
    if (s0 > 0.f && s0 <= __FLT_MAX__) {         // finite range: xmin and xmax are finite
      const float c0 = -xmin * s0;
      for_chunks([&](int) {
#pragma unroll
        for (int u = 0; u < UNITS; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e) atomicAdd(&sh.hist[0][lin_bin(x[u][e], s0, c0)], 1u);
      });
      __syncthreads();
      select_bin(sh.hist[0], sh.bmin[0], sh.bmax[0], need, sh);
      const uint32_t bin0 = sh.sel_bin;
      need = sh.sel_need;
      // round 1: the scores of bin0, in 2048 linear sub-bins with their smallest and largest key
      float s1 = s0 * (float)TK_BINS;
      float c1 = -(xmin + (float)bin0 / s0) * s1;
      if (!(s1 <= __FLT_MAX__ && c1 <= __FLT_MAX__ && c1 >= -__FLT_MAX__)) { s1 = 0.f; c1 = 0.f; }
      for (int i = tid; i < TK_HIST; i += TK_THREADS) sh.hist[0][i] = 0;  // read in select_bin
      for_chunks([&](int) {
#pragma unroll
        for (int u = 0; u < UNITS; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float v = x[u][e];
            if (lin_bin(v, s0, c0) == bin0) {
              const uint32_t b = lin_bin(v, s1, c1);
              const uint32_t kk = score_key(v);
              atomicAdd(&sh.hist[1][b], 1u);
              atomicMin(&sh.bmin[1][b], kk);
              atomicMax(&sh.bmax[1][b], kk);
            }
          }
      });
      __syncthreads();
      select_bin(sh.hist[1], sh.bmin[1], sh.bmax[1], need, sh);
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
      for (int i = tid; i < TK_BINS; i += TK_THREADS) {
        sh.hist[cur ^ 1][i] = 0;
        sh.bmin[cur ^ 1][i] = ALL;
        sh.bmax[cur ^ 1][i] = 0u;
      }
      const float vlo = key_value(lo), vhi = key_value(hi);
      for_chunks([&](int) {
#pragma unroll
        for (int u = 0; u < UNITS; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float v = x[u][e];
            if (v >= vlo && v <= vhi) {
              const uint32_t kk = score_key(v);
              const uint32_t b = (kk - lo) >> shift;
              atomicAdd(&hc[b], 1u);
              atomicMin(&mn[b], kk);
              atomicMax(&mx[b], kk);
            }
          }
      });
      __syncthreads();
      select_bin(hc, mn, mx, need, sh);
      count = sh.sel_count;
      need = sh.sel_need;
      lo = sh.sel_min;
      hi = sh.sel_max;
    }
  } while (false);

  // compaction in index order
  uint32_t gt_chunk = 0, eq_chunk = 0;           // scores above / equal to thr in earlier chunks
  for_chunks([&](int c) {
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
    for (int w = 0; w < TK_WAVES; ++w) {
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
      const int p0 = 4 * (c * CHUNK4 + lane_g + u * WAVE) - off;
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
  });
}

template <int UNITS>
hipError_t launch_rows(const Batch& b, const float* scores, int64_t ld, int k, int32_t* indices,
                       hipStream_t stream) {
  topk_rows<UNITS><<<b.total_q, TK_THREADS, 0, stream>>>(scores, ld, b.cu_q, b.cu_k, b.nseq,
                                                         b.total_q, b.total_k, k, indices);
  return hipGetLastError();
}

}  // namespace

size_t topk_workspace_bytes(const Batch&, int) { return 0; }

hipError_t launch_topk(const Batch& b, const float* scores, int64_t ld, int k, int32_t* indices,
                       void*, hipStream_t stream) {
  // Registers per thread sized for the longest visible row (16-byte groups, plus one for a row
  // that does not start on a 16-byte boundary); rows longer than 32K keys are processed in chunks.
  const int64_t longest = std::min<int64_t>(b.max_k, ld);
  const int64_t groups = (longest + 3) / 4 + 1;
  if (groups <= 1 * TK_THREADS) return launch_rows<1>(b, scores, ld, k, indices, stream);
  if (groups <= 2 * TK_THREADS) return launch_rows<2>(b, scores, ld, k, indices, stream);
  if (groups <= 4 * TK_THREADS) return launch_rows<4>(b, scores, ld, k, indices, stream);
  return launch_rows<8>(b, scores, ld, k, indices, stream);
}

}  // namespace dsa

// Causal per-query top-k ("How GLM5.3 Sparse Attention Affects HBM Memory Usage", How it works /
// Model: top-k 2048, dense below 2K visible tokens, one selection shared by all heads).
//
// Selection rule: the k largest scores among positions 0..p, scores compared as reals
// (-0.0 == +0.0), an equal score going to the lower position; output ascending, -1 padded.
//
// One workgroup of 1024 threads per query row:
//   1. every score becomes an order-preserving 32-bit key (kept in LDS when the row fits);
//      the row's minimum and maximum keys are reduced;
//   2. the threshold key K* (the k-th largest) is found by repeatedly histogramming the keys
//      that fall in the current key interval [lo, hi] into at most 2048 bins of a power-of-two
//      width aligned to lo, and keeping the bin that holds the k-th largest; each round shrinks
//      the interval at least 1024-fold, so at most 3 rounds reach a single key. `need` tracks how many
//      keys equal to K* belong to the selection;
//   3. compaction in index order: each thread owns a contiguous run of positions; a block scan
//      of (count > K*, count == K*) gives every thread its output offset and the number of
//      equal keys before it, so ties are taken lowest-position first.
#include "common.hpp"
#include "kernels.hpp"

namespace dsa {
namespace {

constexpr int TK_THREADS = 1024;
constexpr int TK_WAVES = TK_THREADS / WAVE;
constexpr int TK_BINS = 2048;
constexpr int TK_CACHE = 32768;    // keys kept in LDS (128 KB); longer rows are re-read

struct TopkShared {
  uint32_t hist[TK_BINS];
  uint32_t red_a[TK_WAVES];
  uint32_t red_b[TK_WAVES];
  uint32_t sel_bin;
  uint32_t sel_need;
};

constexpr size_t kTopkLds = TK_CACHE * sizeof(uint32_t) + sizeof(TopkShared);

// Inclusive prefix sums over the block of two counters (all 1024 threads must call).
__device__ __forceinline__ void block_scan2(uint32_t& a, uint32_t& b, uint32_t& tot_a,
                                            uint32_t& tot_b, TopkShared& sh) {
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < WAVE; o <<= 1) {
    const uint32_t ua = __shfl_up(a, o, WAVE);
    const uint32_t ub = __shfl_up(b, o, WAVE);
    if (lane >= o) { a += ua; b += ub; }
  }
  if (lane == WAVE - 1) { sh.red_a[wave] = a; sh.red_b[wave] = b; }
  __syncthreads();
  uint32_t pa = 0, pb = 0;
  tot_a = 0; tot_b = 0;
#pragma unroll
  for (int w = 0; w < TK_WAVES; ++w) {
    const uint32_t ra = sh.red_a[w], rb = sh.red_b[w];
    if (w < wave) { pa += ra; pb += rb; }
    tot_a += ra; tot_b += rb;
  }
  a += pa;
  b += pb;
  __syncthreads();
}

// Calls f(i, key_i) for every position i < n of the row, each thread on positions i == tid
// (mod TK_THREADS) in groups of four. Keys come from the LDS cache when `cached`, otherwise from
// the fp32 scores in global memory with 16-byte loads, unrolled so several loads are in flight.
template <typename F>
__device__ __forceinline__ void scan_row(const float* __restrict__ srow, const uint32_t* keys,
                                         bool cached, int64_t n, F f) {
  const int tid = threadIdx.x;
  const bool vec = cached || ((reinterpret_cast<uintptr_t>(srow) & 15) == 0);
  const int64_t n4 = vec ? (n >> 2) : 0;
  if (cached) {
    const u32x4* k4 = reinterpret_cast<const u32x4*>(keys);
#pragma unroll 4
    for (int64_t j = tid; j < n4; j += TK_THREADS) {
      const u32x4 v = k4[j];
      f(4 * j, v[0]); f(4 * j + 1, v[1]); f(4 * j + 2, v[2]); f(4 * j + 3, v[3]);
    }
  } else {
    const f32x4* s4 = reinterpret_cast<const f32x4*>(srow);
#pragma unroll 4
    for (int64_t j = tid; j < n4; j += TK_THREADS) {
      const f32x4 v = s4[j];
      f(4 * j, score_key(v[0])); f(4 * j + 1, score_key(v[1]));
      f(4 * j + 2, score_key(v[2])); f(4 * j + 3, score_key(v[3]));
    }
  }
  for (int64_t i = 4 * n4 + tid; i < n; i += TK_THREADS)
    f(i, cached ? keys[i] : score_key(srow[i]));
}

__global__ __launch_bounds__(TK_THREADS) void topk_rows(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ cu_q,
    const int64_t* __restrict__ cu_k, int nseq, int total_q, int64_t total_k, int k,
    int32_t* __restrict__ out) {
  extern __shared__ __attribute__((aligned(16))) uint32_t smem[];
  uint32_t* keys = smem;
  TopkShared& sh = *reinterpret_cast<TopkShared*>(smem + TK_CACHE);

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
  const bool cached = n <= TK_CACHE;

  // 1. keys, minimum and maximum
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  scan_row(srow, keys, false, n, [&](int64_t i, uint32_t kk) {
    if (cached) keys[i] = kk;
    kmin = min(kmin, kk);
    kmax = max(kmax, kk);
  });
  kmin = wave_min_u32(kmin);
  kmax = wave_max_u32(kmax);
  if (lane == 0) { sh.red_a[wave] = kmin; sh.red_b[wave] = kmax; }
  __syncthreads();
  kmin = 0xffffffffu;
  kmax = 0u;
#pragma unroll
  for (int w = 0; w < TK_WAVES; ++w) { kmin = min(kmin, sh.red_a[w]); kmax = max(kmax, sh.red_b[w]); }
  __syncthreads();
  auto key_at = [&](int64_t i) -> uint32_t { return cached ? keys[i] : score_key(srow[i]); };

  // 2. threshold key. Bins are 2^shift keys wide, aligned to lo, with the smallest shift that
  // fits [lo, hi] into TK_BINS bins: the bin of a key is one shift and its edges are exact.
  uint64_t lo = kmin, hi = kmax;
  uint32_t need = (uint32_t)k;                   // keys to take from [lo, hi]
  while (lo < hi) {
    const uint64_t span = hi - lo;               // >= 1
    int shift = 0;
    while ((span >> shift) >= TK_BINS) ++shift;
    for (int i = tid; i < TK_BINS; i += TK_THREADS) sh.hist[i] = 0;
    __syncthreads();
    const uint32_t lo32 = (uint32_t)lo, hi32 = (uint32_t)hi;
    scan_row(srow, keys, cached, n, [&](int64_t, uint32_t kk) {
      if (kk >= lo32 && kk <= hi32) atomicAdd(&sh.hist[(kk - lo32) >> shift], 1u);
    });
    __syncthreads();
    const uint32_t h0 = sh.hist[2 * tid], h1 = sh.hist[2 * tid + 1];
    uint32_t incl = h0 + h1, dummy = 0, total = 0, dtot = 0;
    block_scan2(incl, dummy, total, dtot, sh);
    const uint32_t above = total - incl;         // keys in bins above this thread's two bins
    if (above < need && above + h1 >= need) {
      sh.sel_bin = 2 * tid + 1;
      sh.sel_need = need - above;
    } else if (above + h1 < need && above + h1 + h0 >= need) {
      sh.sel_bin = 2 * tid;
      sh.sel_need = need - above - h1;
    }
    __syncthreads();
    const uint64_t bin = sh.sel_bin;
    need = sh.sel_need;
    lo = lo + (bin << shift);
    hi = min(hi, lo + (((uint64_t)1 << shift) - 1));
    __syncthreads();
  }
  const uint32_t kstar = (uint32_t)lo;

  // 3. compaction in index order
  const int64_t per = ((n + TK_THREADS - 1) / TK_THREADS + 3) & ~(int64_t)3;
  const int64_t i0 = min((int64_t)tid * per, n);
  const int64_t i1 = min(i0 + per, n);
  const bool vec = cached || ((reinterpret_cast<uintptr_t>(srow) & 15) == 0);
  auto run = [&](auto&& f) {                     // f(i, key) over this thread's run, in order
    int64_t i = i0;
    if (vec) {
#pragma unroll 4
      for (; i + 4 <= i1; i += 4) {
        if (cached) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(keys + i);
          f(i, v[0]); f(i + 1, v[1]); f(i + 2, v[2]); f(i + 3, v[3]);
        } else {
          const f32x4 v = *reinterpret_cast<const f32x4*>(srow + i);
          f(i, score_key(v[0])); f(i + 1, score_key(v[1]));
          f(i + 2, score_key(v[2])); f(i + 3, score_key(v[3]));
        }
      }
    }
    for (; i < i1; ++i) f(i, key_at(i));
  };
  uint32_t gt = 0, eq = 0;
  run([&](int64_t, uint32_t kk) {
    gt += kk > kstar;
    eq += kk == kstar;
  });
  uint32_t gt_incl = gt, eq_incl = eq, gt_tot = 0, eq_tot = 0;
  block_scan2(gt_incl, eq_incl, gt_tot, eq_tot, sh);
  uint32_t eqc = eq_incl - eq;                   // equal keys before this run
  uint32_t pos = (gt_incl - gt) + min(eqc, need);
  run([&](int64_t i, uint32_t kk) {
    if (kk > kstar) {
      if (pos < (uint32_t)k) orow[pos] = (int32_t)i;
      ++pos;
    } else if (kk == kstar) {
      if (eqc < need) {
        if (pos < (uint32_t)k) orow[pos] = (int32_t)i;
        ++pos;
      }
      ++eqc;
    }
  });
}

}  // namespace

size_t topk_workspace_bytes(const Batch&, int) { return 0; }

hipError_t launch_topk(const Batch& b, const float* scores, int64_t ld, int k, int32_t* indices,
                       void*, hipStream_t stream) {
  hipError_t e = hipFuncSetAttribute((const void*)topk_rows,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kTopkLds);
  if (e != hipSuccess) return e;
  topk_rows<<<b.total_q, TK_THREADS, kTopkLds, stream>>>(scores, ld, b.cu_q, b.cu_k, b.nseq,
                                                         b.total_q, b.total_k, k, indices);
  return hipGetLastError();
}

}  // namespace dsa

// Block-pooled selection ("DeepSeek Sparse Attention" technique page, In the code: MiniMax-M3's
// lightning indexer pools its scores into blocks and keeps the top index_topk_blocks blocks per
// query; GLM-5.3-Flash scores pooled candidates).
//
// A query at position p sees positions 0..p; they are cut into blocks of B consecutive
// positions (the last block holds the remainder). A block's score is the maximum or the mean of
// its visible scores; the topk_blocks best blocks are chosen (an equal score goes to the lower
// block; every block when at most topk_blocks are visible) and the query attends to every
// visible position of the chosen blocks, written ascending and padded with -1 to
// topk_blocks * B. The chosen positions come in runs of B consecutive latent rows, which the
// sparse-MLA gathers read as contiguous memory.
//
// Two kernels (one when the longest row has at most 65536 positions: the select then pools its
// row itself, with the same per-block thread layout and reduction order, so the keys are the
// same bits):
//  * pool: a workgroup per (query, 8192 positions): one sequence lookup, then every thread's
//    eight 16-byte loads of four consecutive scores at once; B/4 adjacent threads per block
//    combine with lane exchanges and each block's order-preserving 32-bit key goes to the
//    workspace [T, ceil(max_seqlen_k / B)].
//  * select: one 1024-thread workgroup per query, the row's block keys staged in LDS. Radix rounds
//    over the offset
//    from the row's smallest key (2048-bin LDS histograms of a power-of-two width fitted to the
//    remaining key range, the bin holding the k-th largest key found with a prefix sum over the
//    bins from the top, at most three rounds) give the threshold key and how many blocks holding
//    it are taken; the chosen blocks are compacted in ascending order through LDS bitmaps of the
//    blocks above and equal to the threshold (two workgroup prefix sums over per-word counts)
//    into an LDS list, from which every thread writes output positions with coalesced stores.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace dsa {
namespace {

constexpr int BT_THREADS = 1024;
constexpr int BT_WAVES = BT_THREADS / WAVE;
constexpr int BT_BINS = 2048;
constexpr int BT_BPT = BT_BINS / BT_THREADS; // histogram bins per thread in the bin search (2)
constexpr int BT_MAX_BLOCKS = 32768;         // block keys of one row staged in LDS (128 KB)
constexpr int BT_MAX_KB = 1024;              // chosen blocks per row
constexpr int POOL_THREADS = 256;

// order-preserving key of the pooled score (-0 and +0 share a key; NaN is not produced)
__device__ __forceinline__ uint32_t pooled_key(float x) { return score_key(x); }

constexpr int POOL_PASSES = 8;               // 16-byte loads per thread, issued together

// grid: x = chunks of POOL_PASSES * POOL_THREADS * 4 positions, y = query rows. One sequence
// lookup per workgroup; B/4 adjacent threads share a block, four positions each, and every
// thread's POOL_PASSES loads go out before the first is used.
template <int B, bool MEAN>
__global__ __launch_bounds__(POOL_THREADS) void block_pool(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ cu_q,
    const int64_t* __restrict__ cu_k, int nseq, int total_q, int64_t total_k, int nb_ld,
    uint32_t* __restrict__ keys) {
  constexpr int TPB = B / 4;                  // threads per block (1..64, a power of two)
  constexpr int CHUNK = POOL_PASSES * POOL_THREADS * 4;   // positions per workgroup
  const int t = blockIdx.y;
  const QueryPos qp = query_pos(cu_q, cu_k, nseq, total_k, t);
  const int64_t n = qp.p >= 0 ? min(min(qp.p + 1, ld), (int64_t)nb_ld * B) : 0;
  const int64_t s_beg = (int64_t)blockIdx.x * CHUNK;
  if (s_beg >= n) return;
  const float* row = scores + (int64_t)t * ld;
  float v[POOL_PASSES][4];
#pragma unroll
  for (int i = 0; i < POOL_PASSES; ++i) {
    const int64_t s0 = s_beg + ((int64_t)i * POOL_THREADS + threadIdx.x) * 4;
    if (s0 + 3 < n) {
      const f32x4 x = *(const f32x4*)(row + s0);
      v[i][0] = x[0]; v[i][1] = x[1]; v[i][2] = x[2]; v[i][3] = x[3];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[i][e] = s0 + e < n ? row[s0 + e] : NAN;   // NaN: not visible
    }
  }
  const int u = threadIdx.x & (TPB - 1);
#pragma unroll
  for (int i = 0; i < POOL_PASSES; ++i) {
    float acc;
    if constexpr (MEAN) {
      acc = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc += v[i][e] == v[i][e] ? v[i][e] : 0.f;
#pragma unroll
      for (int o = 1; o < TPB; o <<= 1) acc += __shfl_xor(acc, o, WAVE);
    } else {
      acc = -INFINITY;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = v[i][e] == v[i][e] ? fmaxf(acc, v[i][e]) : acc;
#pragma unroll
      for (int o = 1; o < TPB; o <<= 1) acc = fmaxf(acc, __shfl_xor(acc, o, WAVE));
    }
    const int64_t s0 = s_beg + ((int64_t)i * POOL_THREADS + threadIdx.x) * 4;  // block start if u == 0
    const int64_t c = s0 / B;
    if (u == 0 && s0 < n) {
      if constexpr (MEAN) acc = acc / (float)min((int64_t)B, n - c * B);
      keys[(int64_t)t * nb_ld + c] = pooled_key(acc);
    }
  }
}

// grid: x = query rows. Writes indices[t, 0 .. kb*B). The row's block keys are staged in LDS and
// every pass over them runs as many steps as the row has blocks (four keys per thread and step,
// loaded before use), so a short row costs a few hundred cycles per pass.
constexpr int BT_UNROLL = 4;
constexpr int BT_STAGE_UNROLL = 8;          // keys per thread and step when staging the row
constexpr int BT_WPT = BT_MAX_BLOCKS / 32 / BT_THREADS;   // bitmap words per thread (1)

// POOL = 0: the block keys come from block_pool's workspace; POOL = 1 (max) or 2 (mean): this
// kernel pools them from the score row itself (rows of at most BT_POOL_MAX positions: one launch
// instead of two, the row's scores read by one workgroup).
constexpr int BT_POOL_PASS = 4;             // 16-byte loads per thread and pooling step
constexpr int BT_POOL_STEP = BT_POOL_PASS * BT_THREADS * 4;   // 16384 positions
constexpr int64_t BT_POOL_MAX = 4 * BT_POOL_STEP;

template <int B, int POOL>
__global__ __launch_bounds__(BT_THREADS) void block_select(
    const uint32_t* __restrict__ keys, const float* __restrict__ scores, int nb_ld, int kb,
    const int32_t* __restrict__ cu_q, const int64_t* __restrict__ cu_k, int nseq, int total_q,
    int64_t total_k, int64_t ld, int32_t* __restrict__ indices) {
  __shared__ uint32_t skey[BT_MAX_BLOCKS];
  __shared__ uint32_t hist[BT_BINS];
  __shared__ uint32_t red[BT_WAVES];
  __shared__ uint32_t above_bits[BT_MAX_BLOCKS / 32];   // blocks above the threshold key
  __shared__ uint32_t equal_bits[BT_MAX_BLOCKS / 32];   // blocks equal to it
  __shared__ uint32_t sel[BT_MAX_KB];        // chosen blocks, ascending
  __shared__ uint32_t bc[4];                 // chosen bin, keys still needed
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = lane_id();
  const QueryPos qp = query_pos(cu_q, cu_k, nseq, total_k, t);
  const int64_t n = qp.p >= 0 ? min(qp.p + 1, ld) : 0;
  // visible blocks (clamped to the keys row, which the host sized to at most BT_MAX_BLOCKS)
  const int nb = (int)min((n + B - 1) / B, (int64_t)nb_ld);
  int32_t* out = indices + (int64_t)t * kb * B;
  const int nout = kb * B;
  if (nb <= kb) {                            // dense: every visible position
    for (int j = tid; j < nout; j += BT_THREADS) out[j] = j < n ? j : -1;
    return;
  }
  constexpr int STEP = BT_THREADS * BT_UNROLL;
  // the row's keys into LDS with their smallest and largest key
  uint32_t kmin = 0xffffffffu, kmax = 0;
  if constexpr (POOL > 0) {
    // pooled here as block_pool does: in each step thread i holds four consecutive positions per
    // pass, B/4 adjacent threads (in one wave) per block, combined with lane exchanges
    constexpr int TPB = B / 4;
    const float* row = scores + (int64_t)t * ld;
    const int u = tid & (TPB - 1);
    for (int64_t p0 = 0; p0 < n; p0 += BT_POOL_STEP) {
      float v[BT_POOL_PASS][4];
#pragma unroll
      for (int i = 0; i < BT_POOL_PASS; ++i) {
        const int64_t s0 = p0 + ((int64_t)i * BT_THREADS + tid) * 4;
        if (s0 + 3 < n) {
          const f32x4 x = *(const f32x4*)(row + s0);
          v[i][0] = x[0]; v[i][1] = x[1]; v[i][2] = x[2]; v[i][3] = x[3];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[i][e] = s0 + e < n ? row[s0 + e] : NAN;   // not visible
        }
      }
#pragma unroll
      for (int i = 0; i < BT_POOL_PASS; ++i) {
        float acc;
        if constexpr (POOL == 2) {
          acc = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) acc += v[i][e] == v[i][e] ? v[i][e] : 0.f;
#pragma unroll
          for (int o = 1; o < TPB; o <<= 1) acc += __shfl_xor(acc, o, WAVE);
        } else {
          acc = -INFINITY;
#pragma unroll
          for (int e = 0; e < 4; ++e) acc = v[i][e] == v[i][e] ? fmaxf(acc, v[i][e]) : acc;
#pragma unroll
          for (int o = 1; o < TPB; o <<= 1) acc = fmaxf(acc, __shfl_xor(acc, o, WAVE));
        }
        const int64_t s0 = p0 + ((int64_t)i * BT_THREADS + tid) * 4;  // block start if u == 0
        const int64_t c = s0 / B;
        if (u == 0 && c < nb) {
          if constexpr (POOL == 2) acc = acc / (float)min((int64_t)B, n - c * B);
          const uint32_t kv = pooled_key(acc);
          skey[c] = kv;
          kmin = min(kmin, kv);
          kmax = max(kmax, kv);
        }
      }
    }
  } else {
  const uint32_t* rk = keys + (int64_t)t * nb_ld;
  for (int c0 = 0; c0 < nb; c0 += BT_THREADS * BT_STAGE_UNROLL) {
    uint32_t kv[BT_STAGE_UNROLL];
#pragma unroll
    for (int u = 0; u < BT_STAGE_UNROLL; ++u) {
      const int c = c0 + u * BT_THREADS + tid;
      kv[u] = c < nb ? rk[c] : 0u;
    }
#pragma unroll
    for (int u = 0; u < BT_STAGE_UNROLL; ++u) {
      const int c = c0 + u * BT_THREADS + tid;
      if (c < nb) {
        skey[c] = kv[u];
        kmin = min(kmin, kv[u]);
        kmax = max(kmax, kv[u]);
      }
    }
  }
  }
  kmin = last_lane(wave_incl_scan(kmin, 0xffffffffu, MinU32()));
  kmax = last_lane(wave_incl_scan(kmax, 0u, MaxU32()));
  if (lane == 0) {
    hist[wave] = kmin;
    hist[BT_WAVES + wave] = kmax;
  }
  __syncthreads();
  kmin = 0xffffffffu;
  kmax = 0;
#pragma unroll
  for (int w = 0; w < BT_WAVES; ++w) {
    kmin = min(kmin, hist[w]);
    kmax = max(kmax, hist[BT_WAVES + w]);
  }
  // Select the kb-th largest key: radix rounds over the offset key - kmin, with 2048 bins of a
  // power-of-two width fitted to the remaining key range (so a row whose keys span a narrow range
  // still spreads over the bins), at most three rounds down to one key. `need` counts the keys
  // still needed from the current range [lo, hi].
  uint32_t lo = kmin, hi = kmax, need = (uint32_t)kb;
  while (lo < hi) {                          // uniform
    const uint64_t range = (uint64_t)(hi - lo) + 1;
    const int sh = max(64 - __builtin_clzll(range - 1) - 11, 0);   // offset bits less 11
    __syncthreads();                         // kmin / kmax or the previous round's bins read
#pragma unroll
    for (int i = 0; i < BT_BPT; ++i) hist[i * BT_THREADS + tid] = 0;
    __syncthreads();
    for (int c0 = 0; c0 < nb; c0 += STEP) {
      uint32_t kv[BT_UNROLL];
#pragma unroll
      for (int u = 0; u < BT_UNROLL; ++u) {
        const int c = c0 + u * BT_THREADS + tid;
        kv[u] = skey[min(c, nb - 1)];
      }
#pragma unroll
      for (int u = 0; u < BT_UNROLL; ++u) {
        const int c = c0 + u * BT_THREADS + tid;
        if (c < nb && kv[u] >= lo && kv[u] <= hi) atomicAdd(&hist[(kv[u] - lo) >> sh], 1u);
      }
    }
    __syncthreads();
    // thread i holds bins 2047 - BT_BPT*i - j, j < BT_BPT (descending key order)
    uint32_t h[BT_BPT], hs = 0;
#pragma unroll
    for (int j = 0; j < BT_BPT; ++j) {
      h[j] = hist[BT_BINS - 1 - BT_BPT * tid - j];
      hs += h[j];
    }
    uint32_t total;
    uint32_t above = wg_exclusive_sum<BT_WAVES>(hs, red, total);
    if (above < need && above + hs >= need) {   // exactly one thread
#pragma unroll
      for (int j = 0; j < BT_BPT; ++j) {
        if (above < need && above + h[j] >= need) {
          bc[0] = BT_BINS - 1 - BT_BPT * tid - j;
          bc[1] = need - above;
        }
        above += h[j];
      }
    }
    __syncthreads();
    const uint32_t bin = bc[0];
    need = bc[1];
    const uint32_t nlo = lo + (bin << sh);
    hi = (uint32_t)min((uint64_t)hi, (uint64_t)nlo + ((uint64_t)1 << sh) - 1);
    lo = nlo;
  }
  const uint32_t thr = lo;                   // the kb-th largest key; `need` blocks equal to it
  // Compaction in ascending block order through two LDS bitmaps (bit c of word c/32): the
  // blocks above the threshold key and those equal to it. Thread i owns the consecutive words
  // BT_WPT*i ..: a workgroup prefix sum over the equal-block counts takes the lowest `need`
  // equal blocks, a second one over the taken counts gives each thread its first output rank,
  // and its taken blocks are written to the list in bit order.
  const int nwords = (nb + 31) / 32;
#pragma unroll
  for (int j = 0; j < BT_WPT; ++j) {
    above_bits[j * BT_THREADS + tid] = 0;
    equal_bits[j * BT_THREADS + tid] = 0;
  }
  __syncthreads();
  for (int c0 = 0; c0 < nb; c0 += STEP) {
    uint32_t kv[BT_UNROLL];
#pragma unroll
    for (int u = 0; u < BT_UNROLL; ++u) kv[u] = skey[min(c0 + u * BT_THREADS + tid, nb - 1)];
#pragma unroll
    for (int u = 0; u < BT_UNROLL; ++u) {
      const int c = c0 + u * BT_THREADS + tid;
      if (c < nb && kv[u] >= thr)
        atomicOr(kv[u] > thr ? &above_bits[c >> 5] : &equal_bits[c >> 5], 1u << (c & 31));
    }
  }
  __syncthreads();
  {
    uint32_t ab[BT_WPT], eb[BT_WPT], ecount = 0;
#pragma unroll
    for (int j = 0; j < BT_WPT; ++j) {
      const int wd = BT_WPT * tid + j;
      ab[j] = wd < nwords ? above_bits[wd] : 0u;
      eb[j] = wd < nwords ? equal_bits[wd] : 0u;
      ecount += __popc(eb[j]);
    }
    uint32_t tot;
    const uint32_t e_before = wg_exclusive_sum<BT_WAVES>(ecount, red, tot);
    // keep the lowest (need - e_before) equal blocks of these words
    // (need - min(..) rather than a subtraction guarded by a comparison, which the compiler
    // marks wrap-free and hoists)
    uint32_t keep = need - min(e_before, need), tcount = 0;
#pragma unroll
    for (int j = 0; j < BT_WPT; ++j) {
      while (keep > 0 && eb[j] != 0) {
        const uint32_t low = eb[j] & (0u - eb[j]);
        ab[j] |= low;
        eb[j] ^= low;
        --keep;
      }
      tcount += __popc(ab[j]);
    }
    uint32_t r = wg_exclusive_sum<BT_WAVES>(tcount, red, tot);
#pragma unroll
    for (int j = 0; j < BT_WPT; ++j) {
      uint32_t word = ab[j];
      while (word != 0) {
        const int bit = __ffs(word) - 1;
        if (r < (uint32_t)kb) sel[r] = (uint32_t)((BT_WPT * tid + j) * 32 + bit);
        ++r;
        word &= word - 1;
      }
    }
  }
  __syncthreads();
  for (int j = tid; j < nout; j += BT_THREADS) {
    const int64_t pos = (int64_t)sel[j / B] * B + (j % B);
    // only the last chosen block can be partial; non-temporal: read by the next launch, so not
    // left dirty in L2 at this one's end
    __builtin_nontemporal_store(pos < n ? (int32_t)pos : -1, out + j);
  }
}

template <int B>
hipError_t launch_block(const Batch& b, const float* scores, int64_t ld, bool mean, int kb,
                        int32_t* indices, void* workspace, hipStream_t stream) {
  const int nb_ld = (int)((b.max_k + B - 1) / B);
  uint32_t* keys = (uint32_t*)workspace;
  if (std::min<int64_t>(b.max_k, ld) <= BT_POOL_MAX) {   // pooled inside the select: one launch
    if (mean)
      block_select<B, 2><<<dim3(b.total_q), BT_THREADS, 0, stream>>>(
          nullptr, scores, nb_ld, kb, b.cu_q, b.cu_k, b.nseq, b.total_q, b.total_k, ld, indices);
    else
      block_select<B, 1><<<dim3(b.total_q), BT_THREADS, 0, stream>>>(
          nullptr, scores, nb_ld, kb, b.cu_q, b.cu_k, b.nseq, b.total_q, b.total_k, ld, indices);
    return hipGetLastError();
  }
  constexpr int CHUNK = POOL_PASSES * POOL_THREADS * 4;
  const dim3 pgrid((unsigned)(((int64_t)nb_ld * B + CHUNK - 1) / CHUNK), b.total_q);
  if (mean)
    block_pool<B, true><<<pgrid, POOL_THREADS, 0, stream>>>(scores, ld, b.cu_q, b.cu_k, b.nseq,
                                                            b.total_q, b.total_k, nb_ld, keys);
  else
    block_pool<B, false><<<pgrid, POOL_THREADS, 0, stream>>>(scores, ld, b.cu_q, b.cu_k, b.nseq,
                                                             b.total_q, b.total_k, nb_ld, keys);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  block_select<B, 0><<<dim3(b.total_q), BT_THREADS, 0, stream>>>(keys, nullptr, nb_ld, kb,
                                                                 b.cu_q, b.cu_k, b.nseq,
                                                                 b.total_q, b.total_k, ld,
                                                                 indices);
  return hipGetLastError();
}

}  // namespace

bool block_topk_supported(const Batch& b, int block, int kb) {
  if (block < 4 || block > 256 || (block & (block - 1)) != 0) return false;
  if (kb < 1 || kb > BT_MAX_KB) return false;
  return (int64_t)(b.max_k + block - 1) / block <= BT_MAX_BLOCKS;
}

size_t block_topk_workspace_bytes(const Batch& b, int block) {
  const int64_t nb_ld = (b.max_k + block - 1) / block;
  return (size_t)b.total_q * (size_t)nb_ld * sizeof(uint32_t);
}

hipError_t launch_block_topk(const Batch& b, const float* scores, int64_t ld, int block,
                             bool mean, int kb, int32_t* indices, void* workspace,
                             hipStream_t stream) {
  switch (block) {
    case 4: return launch_block<4>(b, scores, ld, mean, kb, indices, workspace, stream);
    case 8: return launch_block<8>(b, scores, ld, mean, kb, indices, workspace, stream);
    case 16: return launch_block<16>(b, scores, ld, mean, kb, indices, workspace, stream);
    case 32: return launch_block<32>(b, scores, ld, mean, kb, indices, workspace, stream);
    case 64: return launch_block<64>(b, scores, ld, mean, kb, indices, workspace, stream);
    case 128: return launch_block<128>(b, scores, ld, mean, kb, indices, workspace, stream);
    default: return launch_block<256>(b, scores, ld, mean, kb, indices, workspace, stream);
  }
}

}  // namespace dsa

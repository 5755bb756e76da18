// Shared device helpers for libdsa (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) void lds_void;

constexpr int WAVE = 64;

// D = A(32x16) * B(16x32) + C on the matrix core. Lane l holds A[l%32][8*(l/32)+e] and
// B[8*(l/32)+e][l%32] (e = 0..7); result element r of lane l is D[8*(r/4)+4*(l/32)+r%4][l%32].
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row of the 32x32 MFMA result held in element r of lane l.
__device__ __forceinline__ int mfma32_row(int r, int lane) {
  return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// 64-bit transposing LDS read (gfx950 ds_read_b64_tr_b16). Within each group of 16 lanes,
// lane i receives element (i & 3) of the 4-element chunk addressed by lane 4*e + (i >> 2),
// for e = 0..3. If lane j of the group points at row (j >> 2), columns 4*(j & 3)..+3 of a
// row-major 16-bit matrix, lane i gets column i of those 4 rows.
__device__ __forceinline__ i16x4 lds_read_tr16(const void* lds_ptr) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)((__attribute__((address_space(3))) char*)(lds_void*)lds_ptr));
}

// Eight bf16 from two 4 x 16-bit transposed reads (v0 then v1), reinterpreted as one vector.
__device__ __forceinline__ bf16x8 concat_bf16(i16x4 v0, i16x4 v1) {
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 both = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, both);
}

// Direct global -> LDS copy of 16 bytes per lane. The LDS destination of lane i is
// lds_wave_base + 16*i (lds_wave_base must be wave-uniform); completion is tracked by vmcnt.
__device__ __forceinline__ void global_to_lds16(const void* gptr, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(gptr, (lds_void*)lds_wave_base, 16, 0, 0);
}

// Wait for every outstanding vector-memory, LDS and export operation of this wave.
__device__ __forceinline__ void wait_all_memory() { __builtin_amdgcn_s_waitcnt(0); }

// Wait until at most N vector-memory operations of this wave are outstanding (they complete in
// issue order, so every older one has landed); LDS and export counters are not waited for.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Order-preserving unsigned key of a float score: a > b (as reals) <=> key(a) > key(b).
// -0.0 and +0.0 are the same real number and get the same key.
__device__ __forceinline__ uint32_t score_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (WAVE - 1); }

// Number of set bits of `mask` below this lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o, WAVE));
  return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, WAVE));
  return v;
}

// DPP move of v within the wave; lanes without a source, or outside row_mask, read `identity`.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v, uint32_t identity) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)identity, (int)v, CTRL, ROW_MASK, 0xf, false);
}

// Inclusive scan over the 64 lanes with an associative op and its identity: shifts by 1, 2, 4, 8
// within each row of 16 lanes, then lane 15 of a row is folded into the row above it and lane 31
// into the upper half.
template <typename Op>
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, uint32_t identity, Op op) {
  v = op(v, dpp_u32<0x111>(v, identity));        // row_shr:1
  v = op(v, dpp_u32<0x112>(v, identity));        // row_shr:2
  v = op(v, dpp_u32<0x114>(v, identity));        // row_shr:4
  v = op(v, dpp_u32<0x118>(v, identity));        // row_shr:8
  v = op(v, dpp_u32<0x142, 0xa>(v, identity));   // row_bcast:15 into rows 1 and 3
  v = op(v, dpp_u32<0x143, 0xc>(v, identity));   // row_bcast:31 into rows 2 and 3
  return v;
}

struct AddU32 { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a + b; } };
struct MinU32 { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return min(a, b); } };
struct MaxU32 { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return max(a, b); } };

__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
  return wave_incl_scan(v, 0u, AddU32());
}

// Value of lane 63 (the wave-wide result of an inclusive scan), as a wave-uniform value.
__device__ __forceinline__ uint32_t last_lane(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, WAVE - 1);
}

// Exclusive prefix sum of v over a workgroup of NWAVES waves (every thread calls it); `red` is
// NWAVES words of LDS; also returns the workgroup total. Two barriers.
template <int NWAVES>
__device__ __forceinline__ uint32_t wg_exclusive_sum(uint32_t v, uint32_t* red, uint32_t& total) {
  const int wave = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_scan_u32(v);
  if ((threadIdx.x & (WAVE - 1)) == WAVE - 1) red[wave] = incl;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NWAVES; ++w) {
    const uint32_t x = red[w];
    before += w < wave ? x : 0u;
    tot += x;
  }
  __syncthreads();                            // red may be reused right after
  total = tot;
  return before + incl - v;
}

// Largest b in [0, nseq) with cu[b] <= x (cu ascending, cu[0] <= x).
template <typename I>
__device__ __forceinline__ int find_seq(const I* __restrict__ cu, int nseq, int64_t x) {
  int lo = 0, hi = nseq - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if ((int64_t)cu[mid] <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Same result as find_seq, computed by a whole wave (all 64 lanes must call it with the same x):
// 64 entries are compared per load and the ascending prefix is counted with a ballot, so the
// lookup costs one memory latency per 64 sequences instead of one per bisection step.
template <typename I>
__device__ __forceinline__ int find_seq_wave(const I* __restrict__ cu, int nseq, int64_t x) {
  const int lane = threadIdx.x & (WAVE - 1);
  for (int base = 0;; base += WAVE) {
    const int i = base + 1 + lane;
    const bool le = i < nseq && (int64_t)cu[i] <= x;
    const int cnt = __popcll(__ballot(le));
    if (cnt < WAVE) return base + cnt;
  }
}

// Position of query row t: sequence b, position p (may see 0..p), key base and length.
struct QueryPos {
  int b;
  int64_t p;        // -1 if the row is not a valid query
  int64_t key_base; // first key row of sequence b
  int64_t len;      // L_b
};

// t must be the same for all 64 lanes of the wave (the lookup is a wave-wide ballot). One memory
// round trip per 64 sequences: lane j loads both boundaries of sequence base+j from cu_q and cu_k
// together (index clamped into the arrays, so the loads are unconditional), the ballot over cu_q
// finds the sequence, and its boundaries are read from that lane. The first 64 sequences are
// looked up outside the loop, so the compiler adds no wait there for loads issued before.
__device__ __forceinline__ bool query_pos_step(const int32_t* __restrict__ cu_q,
                                               const int64_t* __restrict__ cu_k, int nseq, int t,
                                               int base, int64_t (&v)[5]) {
  const int lane = threadIdx.x & (WAVE - 1);
  const int j = min(base + lane, max(nseq - 1, 0));
  int32_t qa = cu_q[j], qb = cu_q[j + 1];
  int64_t ka = cu_k[j], kb = cu_k[j + 1];
  // all four loads are issued before the ballot (the compiler would otherwise sink three of them
  // behind it, into a second round trip)
  asm volatile("" : "+v"(qa), "+v"(qb), "+v"(ka), "+v"(kb));
  const bool le = base + lane + 1 < nseq && qb <= t;   // sequence base+lane+1 starts at or before t
  const int cnt = __popcll(__ballot(le));
  if (cnt == WAVE) return false;
  auto rd64 = [&](int64_t x) {
    return (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(x >> 32), cnt) << 32) |
                     (uint32_t)__builtin_amdgcn_readlane((int)x, cnt));
  };
  v[0] = base + cnt;
  v[1] = __builtin_amdgcn_readlane(qa, cnt);
  v[2] = __builtin_amdgcn_readlane(qb, cnt);
  v[3] = rd64(ka);
  v[4] = rd64(kb);
  return true;
}

__device__ __forceinline__ QueryPos query_pos(const int32_t* __restrict__ cu_q,
                                              const int64_t* __restrict__ cu_k, int nseq,
                                              int64_t total_k, int t) {
  int64_t v[5];                                // b, cu_q[b], cu_q[b+1], cu_k[b], cu_k[b+1]
  if (!query_pos_step(cu_q, cu_k, nseq, t, 0, v))
    for (int base = WAVE;; base += WAVE)
      if (query_pos_step(cu_q, cu_k, nseq, t, base, v)) break;
  QueryPos r;
  r.b = (int)v[0];
  int64_t k0 = max((int64_t)0, min(v[3], total_k));
  int64_t k1 = max(k0, min(v[4], total_k));
  r.key_base = k0;
  r.len = k1 - k0;
  const int64_t nq = v[2] - v[1];
  r.p = (t >= v[1] && t < v[2]) ? r.len - nq + (t - v[1]) : -1;
  if (r.p >= r.len) r.p = r.len - 1;
  return r;
}

}  // namespace dsa

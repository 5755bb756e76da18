// Lightning indexer ("How GLM5.3 Sparse Attention Affects HBM Memory Usage", How it works /
// Model): the score of past token s for query t is the weighted sum over indexer heads j of
// ReLU(q_I[t, j] . k_I[s]), one key row per token shared by all heads.
//
// bf16 path (index_head_dim = 128, index_n_heads = 32 * HB): the 32 heads of one query form the
// M dimension of a 32x32x16 MFMA and 32 keys its N dimension, so one MFMA result tile holds
// one query's 32 heads for 32 keys. The epilogue applies ReLU, scales by w and reduces the
// heads inside each lane (16 head rows per lane) plus one cross-lane exchange between the two
// lane halves; lanes 0..31 then hold the 32 finished scores of the tile.
//
//  * decode kernel: few queries per sequence. A workgroup owns 1024 consecutive rows of the
//    flattened key cache; its 4 waves take every fourth 32-key step of each sequence segment in
//    it, so the workgroup reads one contiguous stream. Key rows are loaded coalesced (each load
//    instruction reads four whole rows) into registers two steps ahead and pass through an 8 KB
//    LDS region per wave into the B-operand layout, with the query's heads resident (A
//    operand). Work is laid over the flattened key rows, so ragged batches need no padding.
//  * prefill kernel: many queries per sequence (chunked prefill). A workgroup of 8 waves owns 16
//    queries (2 per wave, A operands in registers) and walks the causal key range in 64-key
//    tiles staged in LDS by direct global->LDS loads through a 4-stage ring (three tiles load
//    while one computes); each B fragment read from LDS feeds both of a wave's queries. Every
//    tile issues the same number of memory operations (masked score stores go to a sink), so
//    the ring is waited on with exact counts.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace dsa {
namespace {

constexpr int D = 128;                  // index_head_dim on the bf16 path

// max(x, 0). This file is compiled without IEEE NaN handling (no NaN reaches the indexer), so
// fmaxf is a single v_max_f32 instead of a NaN-quieting v_max followed by the maximum.
__device__ __forceinline__ float relu(float x) { return fmaxf(x, 0.f); }

// x of lanes l and l^32 added, in every lane, with one gfx950 lane-half swap (of its two
// results one holds the low half of x in both halves, the other the high half).
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
constexpr int DEC_KEYS_PER_WAVE = 256;
constexpr int DEC_WAVES = 4;
constexpr int DEC_KEYS_PER_BLOCK = DEC_KEYS_PER_WAVE * DEC_WAVES;

constexpr int DEC_STEP = 32;            // keys per MFMA step
constexpr int DEC_NSTEP = DEC_KEYS_PER_WAVE / DEC_STEP;   // steps of one wave in a workgroup (8)

// Streams key rows s_beg, s_beg + stride, .. (32-key steps) of one sequence for query t, below
// s_end. Each step's 32 key rows (8 KB) are loaded into registers two steps ahead of the MFMAs,
// so about 16 KB per wave are in flight, and pass through LDS into the B-operand layout.
// With `preloaded`, b0..b2 already hold the first three steps' rows (loaded by flattened row
// before the sequence lookup: rows past the sequence belong to the next one, and their scores
// are computed but never stored).
// NQ > 1 (several new tokens of one sequence, e.g. multi-token prediction): queries t .. t+NQ-1
// share the key stream, each key step multiplied by every query's operands, so a key row is
// read once for all of them; query t+j (j < nvalid) at position p_first + j stores the keys
// below min(s_lim, p_first + j + 1), and s_end (the stream's end) is that bound of the last
// valid query. Queries j >= nvalid compute on query t's operands and store nothing.
template <int HB, int NQ = 1>
__device__ __forceinline__ void decode_segment(const __bf16* __restrict__ q_idx,
                                               const __bf16* __restrict__ k_idx,
                                               const float* __restrict__ w, int t, int nvalid,
                                               int64_t p_first, int64_t s_lim, int64_t kb0,
                                               int64_t s_beg, int64_t s_end,
                                               float* __restrict__ scores, int64_t ld, int stride,
                                               bool preloaded, bf16x8 (&b0)[8], bf16x8 (&b1)[8],
                                               bf16x8 (&b2)[8], bf16x8* __restrict__ xw) {
  constexpr int HI = 32 * HB;
  // The range is wave-uniform; stating it (scalar registers) keeps the step loop on scalar
  // branches, so the compiler's memory-counter waits stay exact: each step waits for its own
  // rows only, with the next two steps' rows still in flight.
  auto uni = [](int64_t x) {
    return (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(x >> 32)) << 32) |
                     (uint32_t)__builtin_amdgcn_readfirstlane((int)x));
  };
  s_beg = uni(s_beg);
  s_end = uni(s_end);
  kb0 = uni(kb0);
  t = __builtin_amdgcn_readfirstlane(t);
  const int lane = lane_id();
  const int half = lane >> 5;
  const int col = lane & 31;

  bf16x8 a[NQ][HB][8];
  float wr[NQ][HB][16];
  int64_t s_q[NQ];                               // store bound of each query
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const int tj = t + (j < nvalid ? j : 0);
    s_q[j] = j < nvalid ? uni(min(s_lim, p_first + j + 1)) : 0;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const __bf16* qr = q_idx + ((int64_t)tj * HI + hb * 32 + col) * D + half * 8;
#pragma unroll
      for (int st = 0; st < 8; ++st) a[j][hb][st] = *(const bf16x8*)(qr + st * 16);
#pragma unroll
      for (int r = 0; r < 16; ++r)
        wr[j][hb][r] = w[(int64_t)tj * HI + hb * 32 + mfma32_row(r, lane)];
    }
  }

  // Key rows are read coalesced: load st of a step covers rows 4*st .. 4*st+3 of its 32, lane l
  // the 16-byte chunk l%16 of row 4*st + l/16. One pass through this wave's LDS region turns
  // them into the B operand (lane (col, half) of MFMA step st: chunk 2*st+half of row col);
  // chunk c of row r sits in slot c ^ (r mod 16), so both passes are free of bank conflicts.
  const __bf16* kb = k_idx + kb0 * D + (lane & 15) * 8;
  auto load = [&](int64_t s0, bf16x8* dst) {
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const int64_t s = min(s0 + 4 * st + (lane >> 4), s_end - 1);
      dst[st] = *(const bf16x8*)(kb + s * D);
    }
  };
  auto step = [&](int64_t s0, const bf16x8* rows) {
    bf16x8 bop[8];
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const int r = 4 * st + (lane >> 4);
      xw[r * 16 + ((lane & 15) ^ (r & 15))] = rows[st];
    }
#pragma unroll
    for (int st = 0; st < 8; ++st) bop[st] = xw[col * 16 + ((2 * st + half) ^ (col & 15))];
    const int64_t s = s0 + col;
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      float v = 0.f;
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        f32x16 acc = {};
#pragma unroll
        for (int st = 0; st < 8; ++st) acc = mfma32x32x16(a[j][hb][st], bop[st], acc);
#pragma unroll
        for (int r = 0; r < 16; ++r) v = fmaf(wr[j][hb][r], relu(acc[r]), v);
      }
      v += __shfl_xor(v, 32, WAVE);
      if (half == 0 && s < s_q[j]) scores[(int64_t)(t + j) * ld + s] = v;
    }
  };
  // three buffers with fixed register names (a rotating copy would wait for the loads), so
  // two steps of key rows stay in flight while one is multiplied
  if (s_beg >= s_end) return;
  if (!preloaded) {
    load(s_beg, b0);
    load(min(s_beg + stride, s_end - 1), b1);
    load(min(s_beg + 2 * stride, s_end - 1), b2);
  }
  // A wave has at most DEC_NSTEP steps in one segment (its share of the workgroup's rows), so the
  // step sequence is unrolled: straight-line code lets the compiler count the loads in flight
  // exactly, and each step waits for its own rows only (as a loop, the merge of its entry and
  // back-edge states made the top of every third step wait for nearly every load in flight).
#pragma unroll
  for (int i = 0; i < DEC_NSTEP; ++i) {
    const int64_t s0 = s_beg + (int64_t)i * stride;
    if (s0 >= s_end) break;                      // uniform
    bf16x8* cur = i % 3 == 0 ? b0 : (i % 3 == 1 ? b1 : b2);
    step(s0, cur);
    if (i + 3 < DEC_NSTEP) load(min(s0 + 3 * stride, s_end - 1), cur);
  }
}

// Boundaries of sequences lane, lane+64, .. as loaded by every lane of a wave for the lookup below.
struct SeqBounds {
  int64_t ka, kz;   // cu_k of the sequence and of the next one
  int32_t qa, qz;   // cu_q likewise
};

__device__ __forceinline__ SeqBounds load_bounds(const int32_t* __restrict__ cu_q,
                                                 const int64_t* __restrict__ cu_k, int nseq,
                                                 int base) {
  const int i = min(base + lane_id(), max(nseq - 1, 0));
  SeqBounds r;
  r.ka = cu_k[i];
  r.kz = cu_k[i + 1];
  r.qa = cu_q[i];
  r.qz = cu_q[i + 1];
  return r;
}

// The sequence holding flattened key row f: its key rows [kb0, kb1) and query rows [q0, q1).
// One round trip per 64 sequences: lane i holds both boundaries of sequence base+i, a ballot over
// cu_k finds the sequence and its boundaries come from that lane. `first` holds the boundaries of
// sequences 0..63 when the caller loaded them earlier (PRELOADED).
struct SeqSpan {
  int64_t kb0, kb1;
  int q0, q1;
};

template <bool PRELOADED>
__device__ __forceinline__ SeqSpan seq_of_row(const int32_t* __restrict__ cu_q,
                                              const int64_t* __restrict__ cu_k, int nseq,
                                              int64_t f, const SeqBounds& first) {
  const int lane = lane_id();
  SeqSpan r{0, 0, 0, 0};
  for (int base = 0;; base += WAVE) {
    SeqBounds sb = (PRELOADED && base == 0) ? first : load_bounds(cu_q, cu_k, nseq, base);
    asm volatile("" : "+v"(sb.ka), "+v"(sb.kz), "+v"(sb.qa), "+v"(sb.qz));
    const bool le = base + lane + 1 < nseq && sb.kz <= f;
    const int cnt = __popcll(__ballot(le));
    if (cnt == WAVE) continue;
    auto rd64 = [&](int64_t x) {
      return (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(x >> 32), cnt) << 32) |
                       (uint32_t)__builtin_amdgcn_readlane((int)x, cnt));
    };
    r.kb0 = rd64(sb.ka);
    r.kb1 = rd64(sb.kz);
    r.q0 = __builtin_amdgcn_readlane(sb.qa, cnt);
    r.q1 = __builtin_amdgcn_readlane(sb.qz, cnt);
    break;
  }
  return r;
}

// Words zero-filled per workgroup of the side job below (16 per thread).
constexpr int ZF_WORDS = 256 * 16;

// Side job of a decode launch: workgroups past the key range (x >= the key blocks, y == 0)
// zero-fill `zero` (the state the next launch of the step needs cleared) and leave. Returns
// true for those workgroups.
__device__ __forceinline__ bool zero_fill_block(const ZeroFill& zero, int64_t total_k,
                                                int keys_per_block) {
  const int64_t kblocks = (total_k + keys_per_block - 1) / keys_per_block;
  if ((int64_t)blockIdx.x < kblocks) return false;
  if (blockIdx.y == 0) {
    const int64_t base = ((int64_t)blockIdx.x - kblocks) * ZF_WORDS + 4 * threadIdx.x;
#pragma unroll
    for (int i = 0; i < ZF_WORDS / 1024; ++i) {
      const int64_t w = base + 1024 * i;
      if (w + 3 < zero.words) *(u32x4*)(zero.p + w) = u32x4{0u, 0u, 0u, 0u};
      else
        for (int64_t j = w; j < zero.words && j < w + 4; ++j) zero.p[j] = 0u;
    }
  }
  return true;
}

// grid: x = flattened key rows / DEC_KEYS_PER_BLOCK (then the zero-fill workgroups), y = group
// of NQ query offsets within its sequence (NQ consecutive new tokens share the key stream).
template <int HB, int NQ>
__global__ __launch_bounds__(256) void indexer_decode_bf16(
    const __bf16* __restrict__ q_idx, const __bf16* __restrict__ k_idx,
    const float* __restrict__ w, const int32_t* __restrict__ cu_q,
    const int64_t* __restrict__ cu_k, int nseq, int total_q, int64_t total_k,
    float* __restrict__ scores, int64_t ld, ZeroFill zero) {
  __shared__ bf16x8 xbuf[DEC_WAVES][DEC_STEP * 16];   // one step of key rows per wave
  if (zero_fill_block(zero, total_k, DEC_KEYS_PER_BLOCK)) return;
  // wave-uniform (a scalar register): the key range and the step loop below are then uniform,
  // so the loop runs on scalar branches and the compiler's memory-counter waits stay exact
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = lane_id();
  const int j = blockIdx.y;
  int64_t f = (int64_t)blockIdx.x * DEC_KEYS_PER_BLOCK;
  const int64_t f_end = min(f + DEC_KEYS_PER_BLOCK, total_k);
  // The sequence lookup's first loads go out first (lane i: both boundaries of sequence i), then
  // the first three steps' key rows of this wave by flattened row (their addresses do not depend
  // on the lookup). Loads complete in issue order, so the lookup resolves without waiting for
  // the rows, and the query operands it selects are requested while the rows stream in.
  const SeqBounds first = load_bounds(cu_q, cu_k, nseq, 0);
  __builtin_amdgcn_sched_barrier(0);           // keep them ahead of the rows
  bf16x8 b0[8], b1[8], b2[8];
  {
    const __bf16* kr = k_idx + (lane & 15) * 8;
    auto pre = [&](int64_t r, bf16x8* dst) {
#pragma unroll
      for (int st = 0; st < 8; ++st)
        dst[st] = *(const bf16x8*)(kr + min(r + 4 * st, total_k - 1) * D);
    };
    const int64_t r0 = f + DEC_STEP * wave + (lane >> 4);
    pre(r0, b0);
    pre(r0 + DEC_STEP * DEC_WAVES, b1);
    pre(r0 + 2 * DEC_STEP * DEC_WAVES, b2);
  }
  // One segment: the rows of the workgroup's range that belong to the sequence of row f.
  // Returns the first row past it, or f_end if the range cannot continue.
  auto segment = [&](auto preloaded) -> int64_t {
    const SeqSpan sp = seq_of_row<decltype(preloaded)::value>(cu_q, cu_k, nseq, f, first);
    const int64_t kb0 = sp.kb0;
    int64_t kb1 = sp.kb1;
    const int q0 = sp.q0, q1 = sp.q1;
    kb1 = min(kb1, total_k);
    if (kb1 <= f || kb0 > f) return f_end;
    const int64_t seg_end = min(f_end, kb1);
    const int nq = q1 - q0;
    const int j0 = j * NQ;                       // first query offset of this group
    if (j0 < nq && q0 + j0 >= 0 && q0 + nq <= total_q) {
      const int t = q0 + j0;
      const int nvalid = min(NQ, nq - j0);
      const int64_t p_first = (kb1 - kb0) - nq + j0;
      const int64_t s_beg = f - kb0;
      const int64_t s_lim = min(seg_end - kb0, ld);
      const int64_t s_end = min(s_lim, p_first + nvalid);
      decode_segment<HB, NQ>(q_idx, k_idx, w, t, nvalid, p_first, s_lim, kb0,
                             s_beg + DEC_STEP * wave, s_end, scores, ld, DEC_STEP * DEC_WAVES,
                             decltype(preloaded)::value, b0, b1, b2, xbuf[wave]);
    }
    return seg_end;
  };
  f = segment(std::true_type{});                 // usually the whole range
  while (f < f_end) f = segment(std::false_type{});
}

// ---------------------------------------------------------------------------------------------
// fp8 (OCP e4m3fn) keys and queries, decode: the same work layout as the bf16 decode kernel with
// 128-byte key rows. One 32x32x64 fp8 MFMA pairs byte e of lane half h of the A and B operands;
// lane (key, h) holds bytes 64h .. 64h+63 of its key row as the operands of the two K steps and
// lane (head, h) the same bytes of its query row, so each lane loads 64 contiguous bytes of its
// row straight into the B layout (no LDS pass). With key scales, the head sum of a key is
// multiplied by its scale (ReLU(s x) = s ReLU(x) for s >= 0).
// ---------------------------------------------------------------------------------------------
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int F8_NSTEP = 4;                 // 32-key steps of one wave in a workgroup
constexpr int F8_NBUF = 3;                  // steps of key rows in flight per wave
constexpr int F8_KEYS_PER_BLOCK = F8_NSTEP * DEC_STEP * DEC_WAVES;

__device__ __forceinline__ f32x16 mfma32x32x64_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// one 32-key step of key rows as held by a lane: 64 bytes of its row and, with key scales, the
// row's scale
struct Fp8Rows {
  u32x4 v[4];
  float sc;
};

__device__ __forceinline__ i32x8 cat8(u32x4 lo, u32x4 hi) {
  return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// NQ: as decode_segment (queries t .. t+NQ-1 share the key stream).
template <int HB, bool SCALED, int NQ = 1>
__device__ __forceinline__ void decode_segment_fp8(const uint8_t* __restrict__ q_idx,
                                                   const uint8_t* __restrict__ k_idx,
                                                   const float* __restrict__ k_scale,
                                                   const float* __restrict__ w, int t,
                                                   int nvalid, int64_t p_first, int64_t s_lim,
                                                   int64_t kb0, int64_t s_beg, int64_t s_end,
                                                   float* __restrict__ scores, int64_t ld,
                                                   int stride, bool preloaded,
                                                   Fp8Rows (&buf)[F8_NBUF]) {
  constexpr int HI = 32 * HB;
  auto uni = [](int64_t x) {
    return (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(x >> 32)) << 32) |
                     (uint32_t)__builtin_amdgcn_readfirstlane((int)x));
  };
  s_beg = uni(s_beg);
  s_end = uni(s_end);
  kb0 = uni(kb0);
  t = __builtin_amdgcn_readfirstlane(t);
  const int lane = lane_id();
  const int half = lane >> 5;
  const int col = lane & 31;

  i32x8 a[NQ][HB][2];
  float wr[NQ][HB][16];
  int64_t s_q[NQ];                               // store bound of each query
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const int tj = t + (j < nvalid ? j : 0);
    s_q[j] = j < nvalid ? uni(min(s_lim, p_first + j + 1)) : 0;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const uint8_t* qr = q_idx + ((int64_t)tj * HI + hb * 32 + col) * D + 64 * half;
      a[j][hb][0] = *(const i32x8*)qr;
      a[j][hb][1] = *(const i32x8*)(qr + 32);
#pragma unroll
      for (int r = 0; r < 16; ++r)
        wr[j][hb][r] = w[(int64_t)tj * HI + hb * 32 + mfma32_row(r, lane)];
    }
  }
  const uint8_t* kb = k_idx + kb0 * D + 64 * half;
  auto load = [&](int64_t s0, Fp8Rows& dst) {
    const int64_t s = min(s0 + col, s_end - 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst.v[i] = *(const u32x4*)(kb + s * D + 16 * i);
    if constexpr (SCALED) dst.sc = k_scale[kb0 + s];
  };
  auto step = [&](int64_t s0, const Fp8Rows& rows) {
    const i32x8 k0 = cat8(rows.v[0], rows.v[1]), k1 = cat8(rows.v[2], rows.v[3]);
    const int64_t s = s0 + col;
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      float v = 0.f;
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        f32x16 acc = mfma32x32x64_fp8(a[j][hb][0], k0, f32x16{});
        acc = mfma32x32x64_fp8(a[j][hb][1], k1, acc);
#pragma unroll
        for (int r = 0; r < 16; ++r) v = fmaf(wr[j][hb][r], relu(acc[r]), v);
      }
      v = halves_sum(v);
      if constexpr (SCALED) v *= rows.sc;
      if (half == 0 && s < s_q[j]) scores[(int64_t)(t + j) * ld + s] = v;
    }
  };
  if (s_beg >= s_end) return;
  if (!preloaded) {
#pragma unroll
    for (int b = 0; b < F8_NBUF; ++b) load(min(s_beg + b * stride, s_end - 1), buf[b]);
  }
  // unrolled, so every buffer index is a compile-time constant (fixed registers)
#pragma unroll
  for (int i = 0; i < F8_NSTEP; ++i) {
    const int64_t s0 = s_beg + (int64_t)i * stride;
    if (s0 >= s_end) break;                      // uniform
    step(s0, buf[i % F8_NBUF]);
    if (i + F8_NBUF < F8_NSTEP) load(min(s0 + F8_NBUF * stride, s_end - 1), buf[i % F8_NBUF]);
  }
}

// grid: x = flattened key rows / F8_KEYS_PER_BLOCK, y = group of NQ query offsets within its
// sequence.
template <int HB, bool SCALED, int NQ>
__global__ __launch_bounds__(256) void indexer_decode_fp8(
    const uint8_t* __restrict__ q_idx, const uint8_t* __restrict__ k_idx,
    const float* __restrict__ k_scale, const float* __restrict__ w,
    const int32_t* __restrict__ cu_q, const int64_t* __restrict__ cu_k, int nseq, int total_q,
    int64_t total_k, float* __restrict__ scores, int64_t ld, ZeroFill zero) {
  if (zero_fill_block(zero, total_k, F8_KEYS_PER_BLOCK)) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = lane_id();
  const int j = blockIdx.y;
  int64_t f = (int64_t)blockIdx.x * F8_KEYS_PER_BLOCK;
  const int64_t f_end = min(f + F8_KEYS_PER_BLOCK, total_k);
  // as in the bf16 kernel: the lookup's loads first, then the first steps' key rows by
  // flattened row
  const SeqBounds first = load_bounds(cu_q, cu_k, nseq, 0);
  __builtin_amdgcn_sched_barrier(0);
  Fp8Rows buf[F8_NBUF];
  {
    const uint8_t* kr = k_idx + 64 * (lane >> 5);
    auto pre = [&](int64_t r, Fp8Rows& dst) {
      r = min(r, total_k - 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) dst.v[i] = *(const u32x4*)(kr + r * D + 16 * i);
      if constexpr (SCALED) dst.sc = k_scale[r];
    };
    const int64_t r0 = f + DEC_STEP * wave + (lane & 31);
#pragma unroll
    for (int b = 0; b < F8_NBUF; ++b) pre(r0 + b * DEC_STEP * DEC_WAVES, buf[b]);
  }
  auto segment = [&](auto preloaded) -> int64_t {
    const SeqSpan sp = seq_of_row<decltype(preloaded)::value>(cu_q, cu_k, nseq, f, first);
    const int64_t kb0 = sp.kb0;
    const int64_t kb1 = min(sp.kb1, total_k);
    if (kb1 <= f || kb0 > f) return f_end;
    const int64_t seg_end = min(f_end, kb1);
    const int nq = sp.q1 - sp.q0;
    const int j0 = j * NQ;
    if (j0 < nq && sp.q0 + j0 >= 0 && sp.q0 + nq <= total_q) {
      const int t = sp.q0 + j0;
      const int nvalid = min(NQ, nq - j0);
      const int64_t p_first = (kb1 - kb0) - nq + j0;
      const int64_t s_beg = f - kb0;
      const int64_t s_lim = min(seg_end - kb0, ld);
      const int64_t s_end = min(s_lim, p_first + nvalid);
      decode_segment_fp8<HB, SCALED, NQ>(q_idx, k_idx, k_scale, w, t, nvalid, p_first, s_lim,
                                         kb0, s_beg + DEC_STEP * wave, s_end, scores, ld,
                                         DEC_STEP * DEC_WAVES, decltype(preloaded)::value, buf);
    }
    return seg_end;
  };
  f = segment(std::true_type{});
  while (f < f_end) f = segment(std::false_type{});
}

constexpr int PF_QW = 2;                // queries per wave
constexpr int PF_WAVES = 8;             // two waves per SIMD: one's MFMAs overlap the other's VALU
constexpr int PF_THREADS = PF_WAVES * WAVE;
constexpr int PF_QB = PF_QW * PF_WAVES; // queries per workgroup
constexpr int PF_KT = 64;               // keys per LDS stage
constexpr int PF_STAGE = PF_KT * D;     // bf16 elements per stage
constexpr int PF_NST = 4;               // stages: three tiles load while one computes
constexpr int PF_LOADS = PF_STAGE * 2 / 16 / PF_THREADS;   // 16-byte loads per thread and tile (2)
constexpr int PF_STORES = 2 * PF_QW;    // score store instructions per wave and tile (4)

// Scores of lanes that have nothing to store (causally masked keys, keys past the row, queries
// past the sequence) go here, one slot per (store, lane) in one of 64 copies picked by the
// workgroup, so that every tile issues the same number of store instructions and the in-order
// memory counter can be waited on exactly. Never read.
constexpr int PF_SINKS = 64;
__device__ float g_score_sink[PF_SINKS * PF_STORES * WAVE];

// grid: x = query blocks of PF_QB over max_seqlen_q, y = sequence, z = key-range splits.
template <int HB>
__global__ __launch_bounds__(PF_THREADS, 1) void indexer_prefill_bf16(
    const __bf16* __restrict__ q_idx, const __bf16* __restrict__ k_idx,
    const float* __restrict__ w, const int32_t* __restrict__ cu_q,
    const int64_t* __restrict__ cu_k, int nseq, int total_q, int64_t total_k,
    float* __restrict__ scores, int64_t ld) {
  constexpr int HI = 32 * HB;
  __shared__ __attribute__((aligned(16))) __bf16 ktile[PF_NST][PF_STAGE];

  const int b = blockIdx.y;
  if (b >= nseq) return;
  const int q0 = cu_q[b];
  const int nq = cu_q[b + 1] - q0;
  // clamped like query_pos(): inconsistent cu_seqlens give wrong scores, never a read outside
  // k_idx
  const int64_t kb0 = max((int64_t)0, min(cu_k[b], total_k));
  const int64_t kb1 = max(kb0, min(cu_k[b + 1], total_k));
  const int64_t L = kb1 - kb0;
  const int jb = blockIdx.x * PF_QB;
  if (jb >= nq || L <= 0 || q0 < 0 || q0 + nq > total_q) return;
  const int jcount = min(PF_QB, nq - jb);
  const int64_t p_first = L - nq + jb;
  const int64_t nkeys = min(min(p_first + jcount, L), ld);   // keys 0..nkeys-1 are needed
  if (nkeys <= 0) return;
  const int64_t ntiles = (nkeys + PF_KT - 1) / PF_KT;
  const int64_t tile_beg = ntiles * blockIdx.z / gridDim.z;
  const int64_t tile_end = ntiles * (blockIdx.z + 1) / gridDim.z;
  if (tile_beg >= tile_end) return;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = lane_id();
  const int half = lane >> 5;
  const int col = lane & 31;

  bf16x8 a[PF_QW][HB][8];
  float wr[PF_QW][HB][16];
#pragma unroll
  for (int qi = 0; qi < PF_QW; ++qi) {
    const int jq = min(jb + wave * PF_QW + qi, nq - 1);
    const int64_t t = q0 + jq;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const __bf16* qr = q_idx + (t * HI + hb * 32 + col) * D + half * 8;
#pragma unroll
      for (int st = 0; st < 8; ++st) a[qi][hb][st] = *(const bf16x8*)(qr + st * 16);
#pragma unroll
      for (int r = 0; r < 16; ++r) wr[qi][hb][r] = w[t * HI + hb * 32 + mfma32_row(r, lane)];
    }
  }

  // The tile loop runs on 32-bit wave-uniform tile numbers (scalar registers). Tiles below
  // t_fast_ld have all 64 key rows in range; tiles below t_fast_st are in range and visible to
  // every query of a full block: those take loads / stores addressed from a uniform base plus a
  // constant per-lane offset, the others clamp and mask per lane.
  const int tb = __builtin_amdgcn_readfirstlane((int)tile_beg);
  const int te = __builtin_amdgcn_readfirstlane((int)tile_end);
  const int t_fast_ld = __builtin_amdgcn_readfirstlane((int)min((int64_t)te, nkeys / PF_KT));
  const int t_fast_st = __builtin_amdgcn_readfirstlane(
      jcount == PF_QB ? (int)min((int64_t)te, min(p_first + 1, nkeys) / PF_KT) : 0);

  // Stage layout: key row r occupies 16 slots of 16 B; the slot of 16-B chunk c is c ^ (r & 15),
  // so any 16 consecutive rows read by one B-operand load use 16 distinct 16-byte bank groups. Tiles past the range
  // load key 0 into their (never read) stage so every iteration issues the same loads.
  uint32_t ld_off[PF_LOADS];                   // byte offset of this lane's chunk in a tile
#pragma unroll
  for (int c = 0; c < PF_LOADS; ++c) {
    const int slot = c * PF_THREADS + tid;
    const int row = slot >> 4;
    ld_off[c] = (uint32_t)(row * D + (((slot & 15) ^ (row & 15)) * 8)) * 2u;
  }
  auto issue = [&](int ti) {
    const int stg = ti & (PF_NST - 1);
    if (__builtin_expect(ti < t_fast_ld, 1)) {
      const char* base = (const char*)(k_idx + (kb0 + (int64_t)ti * PF_KT) * D);
#pragma unroll
      for (int c = 0; c < PF_LOADS; ++c)
        global_to_lds16(base + ld_off[c], &ktile[stg][(c * PF_THREADS + wave * 64) * 8]);
    } else {
#pragma unroll
      for (int c = 0; c < PF_LOADS; ++c) {
        const int slot = c * PF_THREADS + tid;
        const int row = slot >> 4;
        const int gc = (slot & 15) ^ (row & 15);
        const int64_t key = ti < te ? min((int64_t)ti * PF_KT + row, nkeys - 1) : 0;
        global_to_lds16(k_idx + (kb0 + key) * D + gc * 8,
                        &ktile[stg][(c * PF_THREADS + wave * 64) * 8]);
      }
    }
  };
  // one store per (sub, qi) for every lane: both lane halves hold the finished score of key
  // `col` and write it to the same address; lanes without a score write to the sink
  float* sink = g_score_sink + (blockIdx.x % PF_SINKS) * (PF_STORES * WAVE) + lane;
  auto store = [&](auto fast, int ti, int sub, int qi, float v) {
    const int jq = jb + wave * PF_QW + qi;
    if constexpr (decltype(fast)::value) {
      float* row = scores + (int64_t)(q0 + jq) * ld + (int64_t)ti * PF_KT;
      __builtin_nontemporal_store(v, row + (sub * 32 + col));
    } else {
      const int64_t s = (int64_t)ti * PF_KT + sub * 32 + col;
      const int64_t p = p_first + wave * PF_QW + qi;
      const bool own = ti < te && jq < nq && s <= p && s < nkeys;
      float* dst = own ? scores + (int64_t)(q0 + jq) * ld + s : sink + (sub * PF_QW + qi) * WAVE;
      __builtin_nontemporal_store(v, dst);
    }
  };

  // Issue order: the first PF_NST-1 tiles, a full wait, then per iteration [loads of tile
  // ti+3][PF_STORES stores]. From the fourth iteration on, exactly 2*(PF_LOADS+PF_STORES) +
  // PF_STORES memory operations follow the loads of the tile being waited for; in the first
  // three that tile has already landed.
#pragma unroll
  for (int j = 0; j < PF_NST - 1; ++j) issue(tb + j);
  wait_all_memory();

  for (int ti = tb; ti < te; ++ti) {
    const int stg = ti & (PF_NST - 1);
    __builtin_amdgcn_s_waitcnt((((PF_LOADS + PF_STORES) * 2 + PF_STORES) & 15) |
                               ((((PF_LOADS + PF_STORES) * 2 + PF_STORES) >> 4) << 14) |
                               (7 << 4) | (0 << 8));   // vmcnt(16), lgkmcnt(0)
    __syncthreads();                     // tile ti landed for every wave; tile ti-1 consumed
    issue(ti + PF_NST - 1);
    // the exact wait above counts this tile's loads before its stores: keep them in that order
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (HB == 1) {
      // Four MFMA chains per tile, (sub, query) = (0,0) (0,1) (1,0) (1,1). Each chain's eight
      // MFMAs are issued interleaved with the epilogue (ReLU, x w, head sum) of the previous
      // chain, one MFMA to four VALU instructions, so the matrix core stays busy while the
      // epilogue runs; two accumulators alternate. The body is one basic block per tile kind
      // (stores without per-lane masks, or masked), so the interleave is not cut by branches.
      auto body = [&](auto fast) __attribute__((always_inline)) {
        bf16x8 bop[2][8];
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
          const int row = sub * 32 + col;
#pragma unroll
          for (int st = 0; st < 8; ++st) {
            const int chunk = st * 2 + half;
            bop[sub][st] = *(const bf16x8*)&ktile[stg][(row * 16 + (chunk ^ (row & 15))) * 8];
          }
        }
        auto epilogue = [&](int qi, const f32x16& acc) {
          float v = 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) v = fmaf(wr[qi][0][r], relu(acc[r]), v);
          return v;
        };
        f32x16 acc[2];
        float vs[4];
        acc[0] = f32x16{};
#pragma unroll
        for (int st = 0; st < 8; ++st) acc[0] = mfma32x32x16(a[0][0][st], bop[0][st], acc[0]);
#pragma unroll
        for (int c = 1; c < 4; ++c) {
          const int sub = c >> 1, qi = c & 1;
          acc[c & 1] = f32x16{};
#pragma unroll
          for (int st = 0; st < 8; ++st)
            acc[c & 1] = mfma32x32x16(a[qi][0][st], bop[sub][st], acc[c & 1]);
          vs[c - 1] = epilogue((c - 1) & 1, acc[(c - 1) & 1]);
        }
        // schedule (one pattern for the whole body): chain 0 alone, then chains 1..3 with each
        // MFMA followed by four epilogue instructions of the chain before it
#pragma unroll
        for (int st = 0; st < 8; ++st) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
        for (int st = 0; st < 24; ++st) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        }
        vs[3] = epilogue(1, acc[1]);
#pragma unroll
        for (int c = 0; c < 4; ++c) store(fast, ti, c >> 1, c & 1, halves_sum(vs[c]));
      };
      if (__builtin_expect(ti < t_fast_st, 1))
        body(std::true_type{});
      else
        body(std::false_type{});
    } else {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const int row = sub * 32 + col;
        bf16x8 bop[8];
#pragma unroll
        for (int st = 0; st < 8; ++st) {
          const int chunk = st * 2 + half;
          bop[st] = *(const bf16x8*)&ktile[stg][(row * 16 + (chunk ^ (row & 15))) * 8];
        }
#pragma unroll
        for (int qi = 0; qi < PF_QW; ++qi) {
          float v = 0.f;
#pragma unroll
          for (int hb = 0; hb < HB; ++hb) {
            f32x16 acc = {};
#pragma unroll
            for (int st = 0; st < 8; ++st) acc = mfma32x32x16(a[qi][hb][st], bop[st], acc);
#pragma unroll
            for (int r = 0; r < 16; ++r) v = fmaf(wr[qi][hb][r], relu(acc[r]), v);
          }
          if (__builtin_expect(ti < t_fast_st, 1))
            store(std::true_type{}, ti, sub, qi, halves_sum(v));
          else
            store(std::false_type{}, ti, sub, qi, halves_sum(v));
        }
      }
    }
  }
}

// fp32 path: one thread per (query, key); plain FMA loops.
__global__ __launch_bounds__(256) void indexer_f32(
    const float* __restrict__ q_idx, const float* __restrict__ k_idx,
    const float* __restrict__ w, const int32_t* __restrict__ cu_q,
    const int64_t* __restrict__ cu_k, int nseq, int total_q, int64_t total_k, int HI, int DI,
    float* __restrict__ scores, int64_t ld) {
  const int t = blockIdx.y;
  if (t >= total_q) return;
  const QueryPos qp = query_pos(cu_q, cu_k, nseq, total_k, t);
  const int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (qp.p < 0 || s > qp.p || s >= ld) return;
  const float* kr = k_idx + (qp.key_base + s) * DI;
  const float* qt = q_idx + (int64_t)t * HI * DI;
  float acc = 0.f;
  for (int j = 0; j < HI; ++j) {
    float d = 0.f;
    for (int c = 0; c < DI; ++c) d = fmaf(qt[j * DI + c], kr[c], d);
    acc = fmaf(w[(int64_t)t * HI + j], fmaxf(d, 0.f), acc);
  }
  scores[(int64_t)t * ld + s] = acc;
}

}  // namespace

hipError_t launch_indexer_bf16(const Batch& b, const void* q_idx, const void* k_idx,
                               const float* w, int index_n_heads, float* scores, int64_t ld,
                               hipStream_t stream, ZeroFill zero, bool* zeroed) {
  if (zeroed) *zeroed = false;
  const __bf16* q = (const __bf16*)q_idx;
  const __bf16* k = (const __bf16*)k_idx;
  const bool prefill = b.max_q >= PF_QB;
  if (prefill) {
    const int qblocks = (b.max_q + PF_QB - 1) / PF_QB;
    const int64_t base = (int64_t)qblocks * b.nseq;
    int splits = (int)((1024 + base - 1) / base);
    splits = std::max(1, std::min(splits, 8));
    dim3 grid(qblocks, b.nseq, splits);
    if (index_n_heads == 32)
      indexer_prefill_bf16<1><<<grid, PF_THREADS, 0, stream>>>(q, k, w, b.cu_q, b.cu_k, b.nseq,
                                                               b.total_q, b.total_k, scores, ld);
    else
      indexer_prefill_bf16<2><<<grid, PF_THREADS, 0, stream>>>(q, k, w, b.cu_q, b.cu_k, b.nseq,
                                                               b.total_q, b.total_k, scores, ld);
  } else {
    // 32 indexer heads: up to four new tokens of a sequence share one key stream (their
    // operands stay in registers); 64 heads: one token per stream
    const int nq = index_n_heads == 32 ? std::min(b.max_q, 4) : 1;
    const int64_t zblocks = zero.p ? (zero.words + ZF_WORDS - 1) / ZF_WORDS : 0;
    dim3 grid((unsigned)((b.total_k + DEC_KEYS_PER_BLOCK - 1) / DEC_KEYS_PER_BLOCK + zblocks),
              (unsigned)((b.max_q + nq - 1) / nq));
    auto go = [&](auto kern) {
      kern<<<grid, 256, 0, stream>>>(q, k, w, b.cu_q, b.cu_k, b.nseq, b.total_q, b.total_k,
                                     scores, ld, zero);
    };
    if (zeroed) *zeroed = zero.p != nullptr;
    if (index_n_heads == 64) go(indexer_decode_bf16<2, 1>);
    else if (nq == 1) go(indexer_decode_bf16<1, 1>);
    else if (nq == 2) go(indexer_decode_bf16<1, 2>);
    else if (nq == 3) go(indexer_decode_bf16<1, 3>);
    else go(indexer_decode_bf16<1, 4>);
  }
  return hipGetLastError();
}

hipError_t launch_indexer_fp8(const Batch& b, const void* q_idx, const void* k_idx,
                              const float* k_scale, const float* w, int index_n_heads,
                              float* scores, int64_t ld, hipStream_t stream, ZeroFill zero,
                              bool* zeroed) {
  const uint8_t* q = (const uint8_t*)q_idx;
  const uint8_t* k = (const uint8_t*)k_idx;
  // as the bf16 kernel: up to four new tokens of a sequence share one key stream (32 heads)
  const int nq = index_n_heads == 32 ? std::min(b.max_q, 4) : 1;
  const int64_t zblocks = zero.p ? (zero.words + ZF_WORDS - 1) / ZF_WORDS : 0;
  dim3 grid((unsigned)((b.total_k + F8_KEYS_PER_BLOCK - 1) / F8_KEYS_PER_BLOCK + zblocks),
            (unsigned)((b.max_q + nq - 1) / nq));
  auto go = [&](auto kern) {
    kern<<<grid, 256, 0, stream>>>(q, k, k_scale, w, b.cu_q, b.cu_k, b.nseq, b.total_q,
                                   b.total_k, scores, ld, zero);
  };
  if (zeroed) *zeroed = zero.p != nullptr;
  auto by_nq = [&](auto scaled) {
    constexpr bool S = decltype(scaled)::value;
    if (index_n_heads == 64) go(indexer_decode_fp8<2, S, 1>);
    else if (nq == 1) go(indexer_decode_fp8<1, S, 1>);
    else if (nq == 2) go(indexer_decode_fp8<1, S, 2>);
    else if (nq == 3) go(indexer_decode_fp8<1, S, 3>);
    else go(indexer_decode_fp8<1, S, 4>);
  };
  if (k_scale) by_nq(std::true_type{});
  else by_nq(std::false_type{});
  return hipGetLastError();
}

hipError_t launch_indexer_f32(const Batch& b, const float* q_idx, const float* k_idx,
                              const float* w, int index_n_heads, int index_head_dim,
                              float* scores, int64_t ld, hipStream_t stream) {
  dim3 grid((unsigned)((b.max_k + 255) / 256), b.total_q);
  indexer_f32<<<grid, 256, 0, stream>>>(q_idx, k_idx, w, b.cu_q, b.cu_k, b.nseq, b.total_q,
                                        b.total_k, index_n_heads, index_head_dim, scores, ld);
  return hipGetLastError();
}

}  // namespace dsa

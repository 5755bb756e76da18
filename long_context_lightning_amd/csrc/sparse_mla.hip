// Sparse MLA forward in MQA mode ("How GLM5.3 Sparse Attention Affects HBM Memory Usage",
// How it works / Model): every query head attends, with softmax, over only the top-k selected
// latent rows; the key is the full 576-wide latent+rope row and the value its leading 512
// columns (weight absorption), so one gathered 1152-byte row serves all heads for both products.
//
// bf16 kernel: one workgroup = (query, KV split, group of 32 heads), 4 waves, 80 KB of LDS, so
// two workgroups share a CU. The two head groups of one (query, split) sit next to each other
// on one XCD and gather the same rows at about the same time: the second read comes from L2.
//   * Tiles of 64 selected rows are gathered straight from HBM into one LDS stage with direct
//     global->LDS 16-byte loads; the other workgroup on the CU computes while one waits. Each
//     row's 72 chunks of 16 B are stored with the chunk slot XOR-ed by a 3-bit function of the
//     row (swz) that keeps every MFMA operand read free of LDS bank conflicts.
//   * QK^T is computed transposed, S^T[rows x heads] = KV[rows x 576] * Q^T, on 32x32x16 MFMAs:
//     wave (rb, kh) owns rows 32*rb.. and K half kh for all 32 heads; the query half is resident
//     in registers (B operand). The two K-half partial sums of a row block are exchanged through
//     LDS, each wave keeping half of the block's elements, so every lane holds one head.
//   * Softmax in fp32 (base-2 exponent, scale*log2(e) folded into the logits) against a fixed
//     reference maximum per head; P is rounded to bf16 into LDS.
//   * P*V on 32x32x16 MFMAs: wave w owns value columns 128*w.. of all 32 heads; P is the A
//     operand, V (row-major in the same LDS tile) is read column-wise with the gfx950
//     transposing LDS read. The fp32 output block stays in registers across tiles.
//   * With several splits per query, each split stores its normalised partial output in bf16,
//     in the accumulator register layout (32 contiguous bytes per lane and value block), and
//     its log-sum-exp; a combine kernel merges them with exp(lse_i - lse) weights. With one
//     split the output block is transposed through LDS and written with 16-byte stores.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace dsa {
namespace {

constexpr int DQK = 576;
constexpr int DV = 512;
constexpr int HG = 32;                       // heads per workgroup
constexpr int TILE = 64;                     // selected rows per LDS stage
constexpr int ROWB = DQK * 2;                // 1152 bytes per latent row
constexpr int CHUNKS = ROWB / 16;            // 72 chunks of 16 B
constexpr int STAGE_BYTES = TILE * ROWB;     // 73728
constexpr int ROPE_OFF = DV * 2;             // byte offset of the RoPE columns in a row
constexpr int P_STRIDE = TILE + 8;           // bf16 elements per head row of P (padded)
constexpr int OFF_R = STAGE_BYTES;           // 8 KB: QK half-sum exchange, then P
constexpr int R_BYTES = 4 * 8 * 64 * 4;      // 8 floats per lane per wave
constexpr int MLA_LDS = OFF_R + R_BYTES;     // 80 KB: two workgroups per CU
constexpr int LOADS_PER_THREAD = STAGE_BYTES / 16 / 256;   // 18
constexpr int QK_STEPS = DQK / 16 / 2;       // 18 MFMA k-steps per K half
constexpr int VB_WAVE = DV / 32 / 4;         // 4 value blocks of 32 columns per wave
static_assert(LOADS_PER_THREAD * 256 * 16 == STAGE_BYTES, "stage must split evenly");
static_assert(HG * P_STRIDE * 2 <= R_BYTES, "P fits the exchange region");
static_assert(2 * MLA_LDS <= 160 * 1024, "two workgroups per CU");

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kHeadroom = 16.f;            // log2 headroom of a reference maximum

// LDS slot of 16-byte chunk c of tile row r is c ^ swz(r). swz takes all 8 values on every 8
// aligned rows and distinct values on the even and on the odd rows of every 16, so the QK
// operand reads (32 consecutive rows, one chunk) are conflict-free for 32- and 64-bank LDS;
// and within every aligned 4-row block its bits (2,1) take all four values with bit 2 differing
// between rows r and r+2, which makes the transposed V reads (4 rows x 64 bytes) conflict-free.
// The RoPE chunks 64..71 stay in slots 64..71 (the XOR only touches the low 3 bits).
__device__ __forceinline__ int swz(int r) {
  return (2 * (r & 3) + ((r >> 2) & 1)) ^ (((r >> 3) & 1) << 1);
}

// Hides a value from loop-invariant code motion so per-tile address math is recomputed
// instead of occupying registers across the tile loop.
__device__ __forceinline__ void opaque(int& x) { asm volatile("" : "+v"(x)); }

// Softmax statistics live in the RoPE columns of the tile being processed: those columns are
// only read by QK^T, which every wave has finished before the first statistic is written.
// Float i sits in row i/32 at RoPE byte 4*(i%32).
__device__ __forceinline__ float* stat(char* stage, int i) {
  return (float*)(stage + (i >> 5) * ROWB + ROPE_OFF + (i & 31) * 4);
}
constexpr int ST_MAX = 0;       // [4 waves][HG] maximum over each wave's 16 rows
constexpr int ST_SUM = 128;     // [4 waves][HG] sums over the same rows
constexpr int ST_FLAG = 256;    // [4]           wave saw a logit beyond its reference headroom

// Element r of the QK accumulator kept by K-half wave kh after the exchange: value q (0..7) of
// the wave is element 8*(q/4) + 4*kh + q%4; the other eight go to the partner wave.
__device__ __forceinline__ int kept_elem(int q, int kh) { return 8 * (q >> 2) + 4 * kh + (q & 3); }

// grid: 1-D, 8 * ceil(T/8) * nsplit * (H/32) workgroups. Consecutive workgroups are dispatched
// round-robin to the 8 XCDs; the mapping gives every workgroup of one query the same XCD, and
// puts the two head halves of one (query, split) next to each other there, so the second read
// of each gathered row is served by that XCD's L2.
__global__ __launch_bounds__(256, 2) void sparse_mla_bf16(
    const __bf16* __restrict__ q, const __bf16* __restrict__ kv,
    const int32_t* __restrict__ indices, int k, const int32_t* __restrict__ cu_q,
    const int64_t* __restrict__ cu_k, int nseq, int total_q, int64_t total_k, int H,
    float scale_log2, int nsplit, int rows_per_split, int tgroups, __bf16* __restrict__ out,
    float* __restrict__ lse, __bf16* __restrict__ part_o, float* __restrict__ part_lse) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int nhg = H / HG;
  const int xcd = blockIdx.x & 7;
  const int kk = blockIdx.x >> 3;
  const int hg = kk % nhg;
  const int split = (kk / nhg) % nsplit;
  const int t = (kk / nhg / nsplit) * 8 + xcd;
  if (t >= total_q) return;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = lane_id();
  const int half = lane >> 5;
  const int c32 = lane & 31;
  const int kh = wave & 1;        // QK: K half (columns 288*kh ..); softmax: kept element set
  const int rb = wave >> 1;       // QK: row block (rows 32*rb ..)
  const int cq = wave;            // PV: value columns 128*cq ..

  const QueryPos qp = query_pos(cu_q, cu_k, nseq, total_k, t);
  const int64_t L = qp.len;
  const uint32_t Lu = (uint32_t)min(L, (int64_t)0x7fffffff);
  const int r_beg = split * rows_per_split;
  const int r_end = min(k, r_beg + rows_per_split);
  const int ntiles = (qp.p >= 0 && L > 0 && r_end > r_beg) ? (r_end - r_beg + TILE - 1) / TILE : 0;
  const int32_t* irow = indices + (int64_t)t * k;
  const __bf16* kvb = kv + qp.key_base * DQK;
  char* stage = lds;
  float* xch = (float*)(lds + OFF_R);         // [4 waves][8][64]
  __bf16* pl = (__bf16*)(lds + OFF_R);        // [HG][P_STRIDE], after the exchange is read

  // Softmax with a fixed reference maximum per head: the first tile in which a head has a finite
  // logit sets its reference m_ref, and probabilities are exp2(s - m_ref) without rescaling the
  // output block. If a later tile exceeds a reference by more than 2^kHeadroom, the workgroup
  // raises the references and restarts its split (softmax is shift-invariant, so the result is
  // the same). Every update of the output accumulators stays in the MFMA pipe.
  f32x16 o[VB_WAVE];
  float m_ref = -INFINITY, l_run = 0.f;
  auto zero_o = [&]() {                       // 0 x 0 + 0 on the matrix core keeps o in AGPRs
    const bf16x8 z = {};
#pragma unroll
    for (int db = 0; db < VB_WAVE; ++db) o[db] = mfma32x32x16(z, z, f32x16{});
  };
  zero_o();

  if (ntiles > 0) {
    // index of tile row `lane`, -1 past the split
    auto load_idx = [&](int tile) -> int {
      const int r = r_beg + tile * TILE + lane;
      const int v = irow[min(r, k - 1)];
      return (tile < ntiles && r < r_end) ? v : -1;
    };
    // gathers one tile: slot c*256+tid of the stage holds chunk (slot%72)^swz(row) of row
    // slot/72 (invalid rows read row 0 and are masked later)
    auto issue = [&](int idxv) {
      int tt = tid;
      opaque(tt);
#pragma unroll
      for (int g = 0; g < LOADS_PER_THREAD / 6; ++g) {
        int vs[6], gcs[6];
#pragma unroll
        for (int j = 0; j < 6; ++j) {
          const int slot = (g * 6 + j) * 256 + tt;
          const int row = slot / CHUNKS;
          gcs[j] = (slot - row * CHUNKS) ^ swz(row);
          vs[j] = __shfl(idxv, row, WAVE);
        }
#pragma unroll
        for (int j = 0; j < 6; ++j) {
          const uint32_t v = (uint32_t)vs[j] < Lu ? (uint32_t)vs[j] : 0u;
          global_to_lds16(kvb + (size_t)v * DQK + gcs[j] * 8,
                          stage + ((g * 6 + j) * 256 + wave * 64) * 16);
        }
        __builtin_amdgcn_sched_barrier(0);   // keep the groups apart: bounded live registers
      }
    };

    // the first tile's gathers go out as soon as its indices arrive; the query block loads
    // behind them and both are waited for at the top of the first tile
    int idx_cur = load_idx(0);
    wait_all_memory();
    issue(idx_cur);
    bf16x8 qreg[QK_STEPS];
    {
      const __bf16* qr = q + ((int64_t)t * H + hg * HG + c32) * DQK + kh * (QK_STEPS * 16) +
                         half * 8;
#pragma unroll
      for (int i = 0; i < QK_STEPS; ++i) qreg[i] = *(const bf16x8*)(qr + i * 16);
    }
    // A-operand lane bases: step i reads chunk 36*kh + 2*i + half of row 32*rb + c32; with
    // u = 2*kh + i the slot is 8*(4*kh + u/4) + ((2*(u%4) + half) ^ swz): four lane bases plus
    // 128*(i/4) immediates.
    const int sw = swz(c32);
    int abase[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int u = 2 * kh + j;
      abase[j] = (32 * rb + c32) * ROWB + 128 * (4 * kh + (u >> 2)) +
                 (((2 * (u & 3) + half) ^ sw) << 4);
    }

    for (int tile = 0; tile < ntiles; ++tile) {
      const int idx_nxt = load_idx(tile + 1);
      wait_all_memory();                       // this tile's gathers (and the index load)
      __syncthreads();
      const uint64_t vmask = __ballot((uint32_t)idx_cur < Lu);

      // ---- QK^T half sums: S^T[32 rows x 32 heads] over this wave's 288 columns
      f32x16 s = {};
      {
        bf16x8 a[2];
        auto rd = [&](int i, int b) { a[b] = *(const bf16x8*)(stage + abase[i & 3] + (i >> 2) * 128); };
        rd(0, 0);
#pragma unroll
        for (int i = 0; i < QK_STEPS; ++i) {
          if (i + 1 < QK_STEPS) rd(i + 1, (i + 1) & 1);
          s = mfma32x32x16(a[i & 1], qreg[i], s);
        }
      }
      // ---- exchange half sums: keep element set kh, hand the other to the partner wave
#pragma unroll
      for (int qi = 0; qi < 8; ++qi) xch[(wave * 8 + qi) * 64 + lane] = s[kept_elem(qi, kh ^ 1)];
      __syncthreads();
      float sv[8];
      float mx = -INFINITY;
#pragma unroll
      for (int qi = 0; qi < 8; ++qi) {
        const int e = kept_elem(qi, kh);
        const float v = s[e] + xch[((wave ^ 1) * 8 + qi) * 64 + lane];
        const int row = 32 * rb + mfma32_row(e, lane);
        sv[qi] = ((vmask >> row) & 1) ? v * scale_log2 : -INFINITY;
        mx = fmaxf(mx, sv[qi]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, WAVE));
      if (half == 0) *stat(stage, ST_MAX + wave * HG + c32) = mx;
      __syncthreads();                         // the exchange region is free for P from here
      const float m_tile =
          fmaxf(fmaxf(*stat(stage, ST_MAX + 0 * HG + c32), *stat(stage, ST_MAX + 1 * HG + c32)),
                fmaxf(*stat(stage, ST_MAX + 2 * HG + c32), *stat(stage, ST_MAX + 3 * HG + c32)));
      const bool exceed = m_ref != -INFINITY && m_tile > m_ref + kHeadroom;
      if (m_ref == -INFINITY || exceed) m_ref = m_tile;
      const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
      float ls = 0.f;
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        bf16x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // raw v_exp_f32: arguments are <= headroom; results below 2^-126 flush to 0
          const float p = __builtin_amdgcn_exp2f(sv[4 * g + e] - m_use);
          ls += p;
          pk[e] = (__bf16)p;
        }
        const int row0 = 32 * rb + 16 * g + 8 * kh + 4 * half;
        *(bf16x4*)(pl + c32 * P_STRIDE + row0) = pk;
      }
      ls += __shfl_xor(ls, 32, WAVE);
      if (half == 0) *stat(stage, ST_SUM + wave * HG + c32) = ls;
      const bool wave_exceeds = __ballot(exceed) != 0;   // ballot with every lane active
      if (lane == 0) *stat(stage, ST_FLAG + wave) = wave_exceeds ? 1.f : 0.f;
      __syncthreads();
      const bool restart = (*stat(stage, ST_FLAG + 0) + *stat(stage, ST_FLAG + 1) +
                            *stat(stage, ST_FLAG + 2) + *stat(stage, ST_FLAG + 3)) != 0.f;
      if (restart) {                           // uniform across the workgroup: redo the split
        wait_all_memory();
        __syncthreads();
        zero_o();
        l_run = 0.f;
        idx_cur = load_idx(0);
        wait_all_memory();
        issue(idx_cur);
        tile = -1;
        continue;
      }
      l_run += (*stat(stage, ST_SUM + 0 * HG + c32) + *stat(stage, ST_SUM + 1 * HG + c32)) +
               (*stat(stage, ST_SUM + 2 * HG + c32) + *stat(stage, ST_SUM + 3 * HG + c32));

      // ---- O[32 heads x 128 cols] += P[32 heads x 64 rows] * V[64 rows x 128 cols]
      // V[krow][col] for the B operand of value block blk (32 columns), rows 4*rr.. of the
      // lane's k-group: krow = 16*ks + rw0 + 4*rr with rw0 = 8*(g16/2) + j16/4, and chunk(col)
      // = 4*blk + c2 with blk = 4*cq + db. swz(rw0 + 4) = swz(rw0) ^ 1 and both share bit 2
      // (b2), so slot = 4*(blk ^ b2) + (c2 ^ (swz & 3)): per (rr, parity of blk) one lane base,
      // the rest immediate offsets.
      {
        const int g16 = lane >> 4;
        const int j16 = lane & 15;
        const int c2 = 2 * (g16 & 1) + ((j16 & 3) >> 1);
        const int rw0 = 8 * (g16 >> 1) + (j16 >> 2);
        const int sw0 = swz(rw0);
        const int b2 = sw0 >> 2;
        const char* vb[2][2];
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
          const char* pp = stage + (rw0 + 4 * rr) * ROWB + ((c2 ^ ((sw0 ^ rr) & 3)) << 4) +
                           (j16 & 1) * 8;
          vb[rr][0] = pp + 64 * b2;    // even blk: blk ^ b2 = blk + b2
          vb[rr][1] = pp - 64 * b2;    // odd blk:  blk ^ b2 = blk - b2
        }
        const __bf16* pbase = pl + c32 * P_STRIDE + half * 8;
#pragma unroll
        for (int ks = 0; ks < TILE / 16; ++ks) {
          const bf16x8 pa = *(const bf16x8*)(pbase + ks * 16);
#pragma unroll
          for (int db = 0; db < VB_WAVE; ++db) {
            const int blk = VB_WAVE * cq + db;
            const i16x4 v0 = lds_read_tr16(vb[0][db & 1] + ks * 16 * ROWB + (blk << 6));
            const i16x4 v1 = lds_read_tr16(vb[1][db & 1] + ks * 16 * ROWB + (blk << 6));
            o[db] = mfma32x32x16(pa, concat_bf16(v0, v1), o[db]);
          }
        }
      }
      // the stage and P are free once every wave is past this point: next tile's gathers
      __syncthreads();
      if (tile + 1 < ntiles) issue(idx_nxt);
      idx_cur = idx_nxt;
    }
  }

  // ---- epilogue: 1/l per head, normalised output (final or partial) and log-sum-exp
  float* fin = (float*)(lds + OFF_R);          // [0,32): l per head, [32,64): max per head
  __syncthreads();
  if (wave == 0 && half == 0) {
    fin[c32] = l_run;
    fin[HG + c32] = m_ref;
  }
  __syncthreads();
  float inv[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float l = fin[mfma32_row(r, lane)];
    inv[r] = l > 0.f ? 1.f / l : 0.f;
  }
  if (nsplit > 1) {
    // partial output in the accumulator layout: per (wave, value block) each lane stores its
    // 16 values as 32 contiguous bytes, so a wave writes 2 KB contiguous per block
    __bf16* po = part_o + ((((int64_t)t * nsplit + split) * nhg + hg) * 4 + wave) *
                              (VB_WAVE * 1024);
#pragma unroll
    for (int db = 0; db < VB_WAVE; ++db) {
      bf16x8 lo8, hi8;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        lo8[r] = (__bf16)(o[db][r] * inv[r]);
        hi8[r] = (__bf16)(o[db][8 + r] * inv[8 + r]);
      }
      *(bf16x8*)(po + (db * 64 + lane) * 16) = lo8;
      *(bf16x8*)(po + (db * 64 + lane) * 16 + 8) = hi8;
    }
  } else {
    // final output: transpose the [32 heads x 512] block through LDS, then 16-byte stores
    __bf16* ot = (__bf16*)lds;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int hl = mfma32_row(r, lane);
#pragma unroll
      for (int db = 0; db < VB_WAVE; ++db)
        ot[hl * DV + (VB_WAVE * cq + db) * 32 + c32] = (__bf16)(o[db][r] * inv[r]);
    }
    __syncthreads();
    __bf16* ob = out + ((int64_t)t * H + hg * HG) * DV;
#pragma unroll 4
    for (int i = 0; i < HG * DV / 8 / 256; ++i) {
      const int piece = i * 256 + tid;
      *(bf16x8*)(ob + piece * 8) = *(const bf16x8*)(ot + piece * 8);
    }
  }
  if (wave == 0 && half == 0) {
    const float l = fin[c32];
    const float val = l > 0.f ? (fin[HG + c32] + log2f(l)) * kLn2 : -INFINITY;
    const int64_t h = hg * HG + c32;
    if (nsplit == 1) {
      if (lse) lse[(int64_t)t * H + h] = val;
    } else {
      part_lse[((int64_t)t * nsplit + split) * H + h] = val;
    }
  }
}

// Merges the splits of one (query, 32-head group, wave, value block): 64 lanes, each with the
// 16 (head, column) values the sparse kernel's accumulator layout gives it.
// out = sum_i exp(lse_i - lse) * o_i with lse = logsumexp_i lse_i (natural-log units).
__global__ __launch_bounds__(64) void mla_combine(const __bf16* __restrict__ part_o,
                                                  const float* __restrict__ part_lse,
                                                  int nsplit, int H, __bf16* __restrict__ out,
                                                  float* __restrict__ lse) {
  extern __shared__ float wgt[];               // [nsplit][32] merge weights per head
  const int t = blockIdx.x;
  const int y = blockIdx.y;
  const int db = y % VB_WAVE;
  const int w = (y / VB_WAVE) % 4;
  const int hg = y / (VB_WAVE * 4);
  const int nhg = H / HG;
  const int lane = threadIdx.x;
  const int h0 = hg * HG;                      // first head of this group
  // every split's log-sum-exp of the group's 32 heads, one coalesced load per lane and pass
  for (int j = lane; j < nsplit * 32; j += 64)
    wgt[j] = part_lse[((int64_t)t * nsplit + (j >> 5)) * H + h0 + (j & 31)];
  __syncthreads();
  if (lane < 32) {
    float mx = -INFINITY;
    for (int i = 0; i < nsplit; ++i) mx = fmaxf(mx, wgt[i * 32 + lane]);
    float sum = 0.f;
    if (mx != -INFINITY)
      for (int i = 0; i < nsplit; ++i) sum += expf(wgt[i * 32 + lane] - mx);
    const float tot = (mx == -INFINITY) ? -INFINITY : mx + logf(sum);
    for (int i = 0; i < nsplit; ++i) {
      const float li = wgt[i * 32 + lane];
      wgt[i * 32 + lane] = (li == -INFINITY) ? 0.f : expf(li - tot);
    }
    if (lse && w == 0 && db == 0) lse[(int64_t)t * H + h0 + lane] = tot;
  }
  __syncthreads();
  float acc[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  const int64_t stride = (int64_t)nhg * 4 * VB_WAVE * 1024;     // elements per (t, split)
  const __bf16* po = part_o + (int64_t)t * nsplit * stride + ((hg * 4 + w) * VB_WAVE + db) * 1024 +
                     lane * 16;
  auto add = [&](int i, bf16x8 lo8, bf16x8 hi8) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      acc[r] += wgt[i * 32 + mfma32_row(r, lane)] * (float)lo8[r];
      acc[8 + r] += wgt[i * 32 + mfma32_row(8 + r, lane)] * (float)hi8[r];
    }
  };
  int i = 0;
  for (; i + 4 <= nsplit; i += 4) {            // four splits' loads in flight at once
    bf16x8 lo8[4], hi8[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lo8[j] = *(const bf16x8*)(po + (i + j) * stride);
      hi8[j] = *(const bf16x8*)(po + (i + j) * stride + 8);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) add(i + j, lo8[j], hi8[j]);
  }
  for (; i < nsplit; ++i)
    add(i, *(const bf16x8*)(po + i * stride), *(const bf16x8*)(po + i * stride + 8));
  __bf16* ob = out + ((int64_t)t * H + h0) * DV + (VB_WAVE * w + db) * 32 + (lane & 31);
#pragma unroll
  for (int r = 0; r < 16; ++r) ob[(int64_t)mfma32_row(r, lane) * DV] = (__bf16)acc[r];
}

// fp32 path: one workgroup per (query, head); logits of the selected rows live in LDS.
__global__ __launch_bounds__(256) void sparse_mla_f32(
    const float* __restrict__ q, const float* __restrict__ kv,
    const int32_t* __restrict__ indices, int k, const int32_t* __restrict__ cu_q,
    const int64_t* __restrict__ cu_k, int nseq, int total_q, int64_t total_k, int H, int dqk,
    int dv, float scale, float* __restrict__ out, float* __restrict__ lse) {
  extern __shared__ float fsm[];
  float* z = fsm;                 // [k]
  float* qs = fsm + k;            // [dqk]
  __shared__ float red[256 / WAVE];
  const int t = blockIdx.x;
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  const QueryPos qp = query_pos(cu_q, cu_k, nseq, total_k, t);
  const float* qr = q + ((int64_t)t * H + h) * dqk;
  for (int c = tid; c < dqk; c += 256) qs[c] = qr[c];
  __syncthreads();
  const int32_t* irow = indices + (int64_t)t * k;
  const float* kvb = kv + qp.key_base * dqk;
  float mx = -INFINITY;
  for (int s = tid; s < k; s += 256) {
    const int v = irow[s];
    float zz = -INFINITY;
    if (qp.p >= 0 && v >= 0 && v < qp.len) {
      const float* rr = kvb + (int64_t)v * dqk;
      float d = 0.f;
      for (int c = 0; c < dqk; ++c) d = fmaf(qs[c], rr[c], d);
      zz = d * scale;
    }
    z[s] = zz;
    mx = fmaxf(mx, zz);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, WAVE));
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float sum = 0.f;
  for (int s = tid; s < k; s += 256) {
    const float e = (mx == -INFINITY) ? 0.f : expf(z[s] - mx);
    z[s] = e;
    sum += e;
  }
  sum = wave_sum(sum);
  if ((tid & 63) == 0) red[tid >> 6] = sum;
  __syncthreads();
  sum = red[0] + red[1] + red[2] + red[3];
  const float inv = sum > 0.f ? 1.f / sum : 0.f;
  for (int c = tid; c < dv; c += 256) {
    float acc = 0.f;
    for (int s = 0; s < k; ++s) {
      const float p = z[s];
      if (p == 0.f) continue;
      acc = fmaf(p, kvb[(int64_t)irow[s] * dqk + c], acc);
    }
    out[((int64_t)t * H + h) * dv + c] = acc * inv;
  }
  if (lse && tid == 0) lse[(int64_t)t * H + h] = sum > 0.f ? mx + logf(sum) : -INFINITY;
}

}  // namespace

MlaPlan plan_sparse_mla_bf16(const Batch& b, int k, int n_heads) {
  MlaPlan p;
  const int tiles = (k + TILE - 1) / TILE;
  const int64_t wgs = (int64_t)b.total_q * (n_heads / HG);
  const int64_t wgs1 = wgs > 0 ? wgs : 1;
  int nsplit = (int)((512 + wgs1 - 1) / wgs1);          // two workgroups per CU
  nsplit = std::max(1, std::min(nsplit, (tiles + 1) / 2));          // at least 2 tiles per split
  const int tiles_per_split = (tiles + nsplit - 1) / nsplit;
  p.rows_per_split = tiles_per_split * TILE;
  p.nsplit = (k + p.rows_per_split - 1) / p.rows_per_split;
  // per split: log-sum-exp (fp32) and the normalised partial output (bf16) of every head
  p.workspace = p.nsplit > 1 ? (size_t)b.total_q * p.nsplit * n_heads * (sizeof(float) + DV * 2)
                             : 0;
  return p;
}

hipError_t launch_sparse_mla_bf16(const Batch& b, const void* q, const void* kv,
                                  const int32_t* indices, int k, int n_heads, float scale,
                                  void* out, float* lse, void* workspace, const MlaPlan& plan,
                                  hipStream_t stream) {
  hipError_t e = hipFuncSetAttribute((const void*)sparse_mla_bf16,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, MLA_LDS);
  if (e != hipSuccess) return e;
  float* part_lse = nullptr;
  __bf16* part_o = nullptr;
  if (plan.nsplit > 1) {
    part_lse = (float*)workspace;
    part_o = (__bf16*)(part_lse + (size_t)b.total_q * plan.nsplit * n_heads);
  }
  const int tgroups = (b.total_q + 7) / 8;
  const int64_t nblocks = (int64_t)8 * tgroups * plan.nsplit * (n_heads / HG);
  sparse_mla_bf16<<<dim3((unsigned)nblocks), 256, MLA_LDS, stream>>>(
      (const __bf16*)q, (const __bf16*)kv, indices, k, b.cu_q, b.cu_k, b.nseq, b.total_q,
      b.total_k, n_heads, scale * kLog2e, plan.nsplit, plan.rows_per_split, tgroups,
      (__bf16*)out, lse, part_o, part_lse);
  e = hipGetLastError();
  if (e != hipSuccess || plan.nsplit == 1) return e;
  mla_combine<<<dim3(b.total_q, (n_heads / HG) * 4 * VB_WAVE), 64, plan.nsplit * 32 * sizeof(float),
                stream>>>(part_o, part_lse, plan.nsplit, n_heads, (__bf16*)out, lse);
  return hipGetLastError();
}

hipError_t launch_sparse_mla_f32(const Batch& b, const float* q, const float* kv,
                                 const int32_t* indices, int k, int n_heads, int d_qk, int d_v,
                                 float scale, float* out, float* lse, hipStream_t stream) {
  const size_t smem = (size_t)(k + d_qk) * sizeof(float);
  hipError_t e = hipFuncSetAttribute((const void*)sparse_mla_f32,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  sparse_mla_f32<<<dim3(b.total_q, n_heads), 256, smem, stream>>>(
      q, kv, indices, k, b.cu_q, b.cu_k, b.nseq, b.total_q, b.total_k, n_heads, d_qk, d_v,
      scale, out, lse);
  return hipGetLastError();
}

}  // namespace dsa

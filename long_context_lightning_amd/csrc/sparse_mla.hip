// Sparse MLA forward in MQA mode ("How GLM5.3 Sparse Attention Affects HBM Memory Usage",
// How it works / Model): every query head attends, with softmax, over only the top-k selected
// latent rows; the key is the full 576-wide latent+rope row and the value its leading 512
// columns (weight absorption), so one gathered 1152-byte row serves all 64 heads for both
// products.
//
// bf16 kernel: one workgroup = (query, KV split, group of 64 heads), 4 waves.
//   * Tiles of 64 selected rows are gathered straight from HBM into LDS with direct
//     global->LDS 16-byte loads (double-buffered: tile i+1 streams in while tile i computes).
//     Each row's 72 chunks of 16 B are stored with the chunk slot XOR-ed by a 3-bit function
//     of the row (swz) that keeps every MFMA operand read free of LDS bank conflicts.
//   * QK^T is computed transposed, S^T[rows x heads] = KV[rows x 576] * Q^T, on 32x32x16 MFMAs:
//     wave w owns rows 32*(w&1).. and heads 32*(w>>1)..; the query block is resident in
//     registers (B operand) and KV rows are the A operand read from LDS. In this layout each
//     lane holds one head and 16 rows, so the softmax max / sum are in-lane plus one exchange.
//   * Online softmax in fp32 (base-2 exponent, scale*log2(e) folded into the logits); P is
//     rounded to bf16 into LDS.
//   * P*V on 32x32x16 MFMAs: wave w owns heads 32*(w>>1).. and value columns 256*(w&1)..;
//     P is the A operand, V (row-major in the same LDS tile) is read column-wise with the
//     gfx950 transposing LDS read. The fp32 output block stays in registers across tiles.
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
constexpr int HG = 64;                       // heads per workgroup
constexpr int TILE = 64;                     // selected rows per LDS stage
constexpr int ROWB = DQK * 2;                // 1152 bytes per latent row
constexpr int CHUNKS = ROWB / 16;            // 72 chunks of 16 B
constexpr int STAGE_BYTES = TILE * ROWB;     // 73728
constexpr int ROPE_OFF = DV * 2;             // byte offset of the RoPE columns in a row
constexpr int P_STRIDE = TILE + 8;           // bf16 elements per head row of P (padded)
constexpr int OFF_R = 2 * STAGE_BYTES;       // 16 KB: QK half-sum exchange, then P
constexpr int R_BYTES = 16384;
constexpr int MLA_LDS = OFF_R + R_BYTES;     // 160 KB
constexpr int LOADS_PER_THREAD = STAGE_BYTES / 16 / 256;   // 18
constexpr int QK_STEPS = DQK / 16 / 2;       // 18 MFMA k-steps per K half
static_assert(LOADS_PER_THREAD * 256 * 16 == STAGE_BYTES, "stage must split evenly");
static_assert(HG * P_STRIDE * 2 <= R_BYTES && 4 * 16 * 64 * 4 == R_BYTES, "R region");
static_assert(MLA_LDS <= 160 * 1024, "LDS budget");

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

// s_waitcnt vmcnt(N) with the other counters left alone (GFX9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Softmax statistics live in the RoPE columns of the tile being processed: those columns are
// only read by QK^T, which every wave has finished before the first statistic is written.
// Float i sits in row i/32 at RoPE byte 4*(i%32).
__device__ __forceinline__ float* stat(char* stage, int i) {
  return (float*)(stage + (i >> 5) * ROWB + ROPE_OFF + (i & 31) * 4);
}
constexpr int ST_MAX = 0;       // [2][HG] per row-block tile maximum
constexpr int ST_SUM = 128;     // [2][HG] per row-block tile sum
constexpr int ST_FLAG = 256;    // [4]     wave saw a tile beyond its reference headroom

// grid: 1-D, 8 * ceil(T/8) * nsplit * (H/64) workgroups. Consecutive workgroups are dispatched
// round-robin to the 8 XCDs; the mapping below gives all splits of one query the same XCD so
// its query block is fetched into that XCD's L2 once.
__global__ __launch_bounds__(256, 1) void sparse_mla_bf16(
    const __bf16* __restrict__ q, const __bf16* __restrict__ kv,
    const int32_t* __restrict__ indices, int k, const int32_t* __restrict__ cu_q,
    const int64_t* __restrict__ cu_k, int nseq, int total_q, int64_t total_k, int H,
    float scale_log2, int nsplit, int rows_per_split, int tgroups, __bf16* __restrict__ out,
    float* __restrict__ lse, __bf16* __restrict__ part_o, float* __restrict__ part_lse) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int xcd = blockIdx.x & 7;
  const int kk = blockIdx.x >> 3;
  const int split = kk % nsplit;
  const int rest = kk / nsplit;
  const int t = (rest % tgroups) * 8 + xcd;
  const int hg = rest / tgroups;
  if (t >= total_q) return;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = lane_id();
  const int half = lane >> 5;
  const int c32 = lane & 31;
  const int kh = wave & 1;        // QK: K half (columns 288*kh ..)
  const int hb = wave >> 1;       // QK and PV: head block within the group
  const int rb = kh;              // after the half-sum exchange: row block owned
  const int dvh = wave & 1;       // PV: value-column half
  const int head_lane = hb * 32 + c32;   // head (within the group) of this lane's softmax stats

  const QueryPos qp = query_pos(cu_q, cu_k, nseq, total_k, t);
  const int64_t L = qp.len;
  const uint32_t Lu = (uint32_t)min(L, (int64_t)0x7fffffff);
  const int r_beg = split * rows_per_split;
  const int r_end = min(k, r_beg + rows_per_split);
  const int ntiles = (qp.p >= 0 && L > 0 && r_end > r_beg) ? (r_end - r_beg + TILE - 1) / TILE : 0;
  const int32_t* irow = indices + (int64_t)t * k;
  const __bf16* kvb = kv + qp.key_base * DQK;
  __bf16* pl = (__bf16*)(lds + OFF_R);        // [HG][P_STRIDE]
  float* xch = (float*)(lds + OFF_R);         // [4 waves][16][64]

  // Softmax with a fixed reference maximum per head: the first tile in which a head has a finite
  // logit sets its reference m_ref, and probabilities are exp2(s - m_ref) without rescaling the
  // output block. If a later tile exceeds a reference by more than 2^kHeadroom, the workgroup
  // raises the references and restarts its split (softmax is shift-invariant, so the result is
  // the same). This keeps every update of the output accumulators inside the MFMA pipe.
  f32x16 o[8];
  float m_ref = -INFINITY, l_run = 0.f;

  if (ntiles > 0) {
    // index of tile row `lane`; always issues one load so the vmcnt bookkeeping is uniform
    auto load_idx = [&](int tile) -> int {
      const int r = r_beg + tile * TILE + lane;
      const int v = irow[min(r, k - 1)];
      return (tile < ntiles && r < r_end) ? v : -1;
    };
    // gathers one tile: slot c*256+tid of the stage holds chunk (slot%72)^swz(row) of row
    // slot/72; always issues LOADS_PER_THREAD loads (invalid rows read row 0, masked later)
    auto issue = [&](int idxv, int stg) {
      char* base = lds + stg * STAGE_BYTES;
      int tt = tid;
      opaque(tt);                            // recomputed per tile instead of held in registers
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
                          base + ((g * 6 + j) * 256 + wave * 64) * 16);
        }
        __builtin_amdgcn_sched_barrier(0);   // keep the groups apart: bounded live registers
      }
    };

    const int idx0 = load_idx(0);
    const int idx1 = load_idx(1);
    issue(idx0, 0);                          // tile 0 in flight before the query block loads
    bf16x8 qreg[QK_STEPS];
    {
      const __bf16* qr = q + ((int64_t)t * H + hg * HG + head_lane) * DQK +
                         kh * (QK_STEPS * 16) + half * 8;
#pragma unroll
      for (int i = 0; i < QK_STEPS; ++i) qreg[i] = *(const bf16x8*)(qr + i * 16);
    }
    // A-operand lane bases: step i of this wave reads chunk 36*kh + 2*i + half of rows c32 and
    // 32 + c32 (same swizzle); with u = 2*kh + i the slot is
    // 8*(4*kh + u/4) + ((2*(u%4) + half) ^ swz): four lane bases plus 128*(i/4) immediates.
    const int sw = swz(c32);
    int abase[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int u = 2 * kh + j;
      abase[j] = c32 * ROWB + 128 * (4 * kh + (u >> 2)) + (((2 * (u & 3) + half) ^ sw) << 4);
    }

    // zeroes the output block with MFMAs (0 x 0 + 0) so every definition of o stays in the
    // matrix-core register class
    auto zero_o = [&]() {
      const bf16x8 z = {};
#pragma unroll
      for (int db = 0; db < 8; ++db) o[db] = mfma32x32x16(z, z, f32x16{});
    };
    zero_o();
    issue(idx1, 1);                          // tiles 0 and 1 in flight before the loop
    int idx_cur = idx1;                      // indices of the newest issued tile
    int idx_next = load_idx(2);

    for (int tile = 0; tile < ntiles; ++tile) {
      const int stg = tile & 1;
      if (tile == 0) wait_vmcnt<LOADS_PER_THREAD + 1>();   // tile 1 and idx 2 may be in flight
      else wait_vmcnt<1>();                                // the next index load may be in flight
      __syncthreads();                       // tile rows landed; previous tile fully consumed
      const int idx_tile = tile == 0 ? idx0 : (tile == 1 ? idx1 : idx_cur);
      // The next tile's gathers go out one per QK step (below) so the wave never stalls on a
      // burst of 18 loads; their row indices are fetched from the index register first.
      const bool do_issue = tile >= 1 && tile + 1 < ntiles;
      int tt = tid;
      opaque(tt);
      int nv[LOADS_PER_THREAD];
      if (do_issue) {
#pragma unroll
        for (int c = 0; c < LOADS_PER_THREAD; ++c)
          nv[c] = __shfl(idx_next, (c * 256 + tt) / CHUNKS, WAVE);
      }
      char* nbase = lds + (stg ^ 1) * STAGE_BYTES;
      auto issue_one = [&](int c) {
        const int slot = c * 256 + tt;
        const int row = slot / CHUNKS;
        const int gc = (slot - row * CHUNKS) ^ swz(row);
        const uint32_t v = (uint32_t)nv[c] < Lu ? (uint32_t)nv[c] : 0u;
        global_to_lds16(kvb + (size_t)v * DQK + gc * 8, nbase + (c * 256 + wave * 64) * 16);
      };
      char* sbase = lds + stg * STAGE_BYTES;
      const uint64_t vmask =
          __ballot(r_beg + tile * TILE + lane < r_end && (uint32_t)idx_tile < Lu);

      // ---- QK^T half sums: S^T[64 rows x 32 heads] over this wave's 288 columns
      f32x16 s0 = {}, s1 = {};
      {
        bf16x8 a0[2], a1[2];
        auto rd = [&](int i, int b) {
          const char* pa = sbase + abase[i & 3] + (i >> 2) * 128;
          a0[b] = *(const bf16x8*)pa;
          a1[b] = *(const bf16x8*)(pa + 32 * ROWB);
        };
        static_assert(QK_STEPS == LOADS_PER_THREAD, "one gather per QK step");
        rd(0, 0);
#pragma unroll
        for (int i = 0; i < QK_STEPS; ++i) {
          if (i + 1 < QK_STEPS) rd(i + 1, (i + 1) & 1);
          if (do_issue) issue_one(i);
          s0 = mfma32x32x16(a0[i & 1], qreg[i], s0);
          s1 = mfma32x32x16(a1[i & 1], qreg[i], s1);
        }
      }
      if (tile >= 1) {
        if (do_issue) idx_cur = idx_next;
        idx_next = load_idx(tile + 2);
      }
      // ---- exchange half sums: keep row block kh, hand the other to the partner wave
      const f32x16 give = kh ? s0 : s1;
      f32x16 s = kh ? s1 : s0;
#pragma unroll
      for (int r = 0; r < 16; ++r) xch[(wave * 16 + r) * 64 + lane] = give[r];
      __syncthreads();
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] += xch[((wave ^ 1) * 16 + r) * 64 + lane];

      float sv[16];
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = rb * 32 + mfma32_row(r, lane);
        sv[r] = ((vmask >> row) & 1) ? s[r] * scale_log2 : -INFINITY;
        mx = fmaxf(mx, sv[r]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, WAVE));
      if (half == 0) *stat(sbase, ST_MAX + rb * HG + head_lane) = mx;
      __syncthreads();
      const float m_tile =
          fmaxf(*stat(sbase, ST_MAX + head_lane), *stat(sbase, ST_MAX + HG + head_lane));
      const bool exceed = m_ref != -INFINITY && m_tile > m_ref + kHeadroom;
      if (m_ref == -INFINITY || exceed) m_ref = m_tile;
      const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
      float ls = 0.f;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // raw v_exp_f32: arguments are <= headroom; results below 2^-126 flush to 0
          const float p = __builtin_amdgcn_exp2f(sv[4 * g + e] - m_use);
          ls += p;
          pk[e] = (__bf16)p;
        }
        const int row0 = rb * 32 + 8 * g + 4 * half;
        *(bf16x4*)(pl + head_lane * P_STRIDE + row0) = pk;
      }
      ls += __shfl_xor(ls, 32, WAVE);
      if (half == 0) *stat(sbase, ST_SUM + rb * HG + head_lane) = ls;
      const bool wave_exceeds = __ballot(exceed) != 0;   // ballot with every lane active
      if (lane == 0) *stat(sbase, ST_FLAG + wave) = wave_exceeds ? 1.f : 0.f;
      __syncthreads();
      const bool restart = (*stat(sbase, ST_FLAG + 0) + *stat(sbase, ST_FLAG + 1) +
                            *stat(sbase, ST_FLAG + 2) + *stat(sbase, ST_FLAG + 3)) != 0.f;
      if (restart) {                       // uniform across the workgroup: redo the split
        wait_all_memory();                 // drain this pass's gathers before reusing stages
        __syncthreads();
        zero_o();
        l_run = 0.f;
        issue(idx0, 0);
        issue(idx1, 1);
        idx_cur = idx1;
        idx_next = load_idx(2);
        tile = -1;
        continue;
      }
      l_run += *stat(sbase, ST_SUM + head_lane) + *stat(sbase, ST_SUM + HG + head_lane);

      // ---- O[32 heads x 256 cols] += P[32 heads x 64 rows] * V[64 rows x 256 cols]
      // V[krow][col] for the B operand of value block db (32 columns), rows 4*rr.. of the
      // lane's k-group: krow = 16*ks + rw0 + 4*rr with rw0 = 8*(g16/2) + j16/4, and chunk(col)
      // = 4*blk + c2 with blk = 8*dvh + db. swz(rw0 + 4) = swz(rw0) ^ 1 and both share bit 2
      // (b2), so slot = 4*(blk ^ b2) + (c2 ^ (swz & 3)): per (rr, parity of blk) one lane
      // base, the rest immediate offsets.
      const int g16 = lane >> 4;
      const int j16 = lane & 15;
      const int c2 = 2 * (g16 & 1) + ((j16 & 3) >> 1);
      const int rw0 = 8 * (g16 >> 1) + (j16 >> 2);
      const int sw0 = swz(rw0);
      const int b2 = sw0 >> 2;
      const char* vb[2][2];
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        const char* p = sbase + (rw0 + 4 * rr) * ROWB + ((c2 ^ ((sw0 ^ rr) & 3)) << 4) +
                        (j16 & 1) * 8;
        vb[rr][0] = p + 64 * b2;     // even blk: blk ^ b2 = blk + b2
        vb[rr][1] = p - 64 * b2;     // odd blk:  blk ^ b2 = blk - b2
      }
      const __bf16* pbase = pl + head_lane * P_STRIDE + half * 8;
#pragma unroll
      for (int ks = 0; ks < TILE / 16; ++ks) {
        const bf16x8 pa = *(const bf16x8*)(pbase + ks * 16);
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          const int blk = 8 * dvh + db;
          const i16x4 v0 = lds_read_tr16(vb[0][db & 1] + ks * 16 * ROWB + (blk << 6));
          const i16x4 v1 = lds_read_tr16(vb[1][db & 1] + ks * 16 * ROWB + (blk << 6));
          o[db] = mfma32x32x16(pa, concat_bf16(v0, v1), o[db]);
        }
      }
    }
  } else {
    const bf16x8 z = {};
#pragma unroll
    for (int db = 0; db < 8; ++db) o[db] = mfma32x32x16(z, z, f32x16{});
  }

  // ---- epilogue: 1/l per head, normalised output (final or partial) and log-sum-exp
  float* fin = (float*)(lds + OFF_R);          // [0,64): l per head, [64,128): max per head
  __syncthreads();                             // every wave is done with the stages and P
  if (kh == 0 && half == 0) {
    fin[head_lane] = l_run;
    fin[HG + head_lane] = m_ref;
  }
  __syncthreads();
  float inv[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float l = fin[hb * 32 + mfma32_row(r, lane)];
    inv[r] = l > 0.f ? 1.f / l : 0.f;
  }
  if (nsplit > 1) {
    // partial output in the accumulator layout: per (wave, value block) each lane stores its
    // 16 values as 32 contiguous bytes, so a wave writes 2 KB contiguous per block
    __bf16* po =
        part_o + ((((int64_t)t * nsplit + split) * (H / HG) + hg) * 4 + wave) * (8 * 1024);
#pragma unroll
    for (int db = 0; db < 8; ++db) {
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
    // final output: transpose the [64 heads x 512] block through LDS, then 16-byte stores
    __bf16* ot = (__bf16*)lds;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int hl = hb * 32 + mfma32_row(r, lane);
#pragma unroll
      for (int db = 0; db < 8; ++db)
        ot[hl * DV + dvh * 256 + db * 32 + c32] = (__bf16)(o[db][r] * inv[r]);
    }
    __syncthreads();
    __bf16* ob = out + ((int64_t)t * H + hg * HG) * DV;
#pragma unroll 4
    for (int i = 0; i < HG * DV / 8 / 256; ++i) {
      const int piece = i * 256 + tid;
      *(bf16x8*)(ob + piece * 8) = *(const bf16x8*)(ot + piece * 8);
    }
  }
  if (kh == 0 && dvh == 0 && half == 0) {
    const float l = fin[head_lane];
    const float val = l > 0.f ? (fin[HG + head_lane] + log2f(l)) * kLn2 : -INFINITY;
    const int64_t h = hg * HG + head_lane;
    if (nsplit == 1) {
      if (lse) lse[(int64_t)t * H + h] = val;
    } else {
      part_lse[((int64_t)t * nsplit + split) * H + h] = val;
    }
  }
}

// Merges the splits of one (query, head group, wave block, value block): 64 lanes, each with the
// 16 (head, column) values the sparse kernel's accumulator layout gives it.
// out = sum_i exp(lse_i - lse) * o_i with lse = logsumexp_i lse_i (natural-log units).
__global__ __launch_bounds__(64) void mla_combine(const __bf16* __restrict__ part_o,
                                                  const float* __restrict__ part_lse,
                                                  int nsplit, int H, __bf16* __restrict__ out,
                                                  float* __restrict__ lse) {
  extern __shared__ float wgt[];               // [nsplit][32] merge weights per head
  const int t = blockIdx.x;
  const int y = blockIdx.y;
  const int db = y & 7;
  const int w = (y >> 3) & 3;
  const int hg = y >> 5;
  const int hb = w >> 1, dvh = w & 1;
  const int lane = threadIdx.x;
  const int h0 = hg * HG + hb * 32;            // first head of this block
  // every split's log-sum-exp of the block's 32 heads, one coalesced load per lane and pass
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
    if (lse && dvh == 0 && db == 0) lse[(int64_t)t * H + h0 + lane] = tot;
  }
  __syncthreads();
  float acc[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  const int64_t stride = (int64_t)(H / HG) * 4 * 8 * 1024;      // elements per (t, split)
  const __bf16* po = part_o + (int64_t)t * nsplit * stride + ((hg * 4 + w) * 8 + db) * 1024 +
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
  __bf16* ob =
      out + ((int64_t)t * H + hg * HG + hb * 32) * DV + dvh * 256 + db * 32 + (lane & 31);
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
  int nsplit = (int)((256 + wgs1 - 1) / wgs1);
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
  mla_combine<<<dim3(b.total_q, (n_heads / HG) * 32), 64, plan.nsplit * 32 * sizeof(float),
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

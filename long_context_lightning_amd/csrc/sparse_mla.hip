// Sparse MLA forward in MQA mode ("How GLM5.3 Sparse Attention Affects HBM Memory Usage",
// How it works / Model): every query head attends, with softmax, over only the top-k selected
// latent rows; the key is the full 576-wide latent+rope row and the value its leading 512
// columns (weight absorption), so one gathered 1152-byte row serves all 64 heads for both
// products.
//
// bf16 kernel: one workgroup = (query, KV split, group of 64 heads), 4 waves.
//   * Tiles of 64 selected rows are gathered straight from HBM into LDS with direct
//     global->LDS 16-byte loads (double-buffered: tile i+1 streams in while tile i computes).
//     Each row's 72 chunks of 16 B are stored with the chunk slot XOR-ed by (row & 7) so the
//     MFMA operand reads of 32 consecutive rows hit distinct LDS banks.
//   * QK^T is computed transposed, S^T[rows x heads] = KV[rows x 576] * Q^T, on 32x32x16 MFMAs:
//     wave w owns rows 32*(w&1).. and heads 32*(w>>1)..; the query block is resident in
//     registers (B operand) and KV rows are the A operand read from LDS. In this layout each
//     lane holds one head and 16 rows, so the softmax max / sum are in-lane plus one exchange.
//   * Online softmax in fp32 (base-2 exponent, scale*log2(e) folded into the logits); P is
//     rounded to bf16 into LDS.
//   * P*V on 32x32x16 MFMAs: wave w owns heads 32*(w>>1).. and value columns 256*(w&1)..;
//     P is the A operand, V (row-major in the same LDS tile) is read column-wise with the
//     gfx950 transposing LDS read. The fp32 output block stays in registers across tiles.
//   * With several splits per query, each split writes its normalised partial output and
//     log-sum-exp; a combine kernel merges them with exp(lse_i - lse) weights.
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
constexpr int P_STRIDE = TILE + 8;           // bf16 elements per head row of P (padded)
constexpr int OFF_P = 2 * STAGE_BYTES;
constexpr int OFF_XMAX = OFF_P + HG * P_STRIDE * 2;
constexpr int OFF_XSUM = OFF_XMAX + 2 * HG * 4;
constexpr int OFF_ALPHA = OFF_XSUM + 2 * HG * 4;
constexpr int MLA_LDS = OFF_ALPHA + HG * 4;
constexpr int LOADS_PER_THREAD = STAGE_BYTES / 16 / 256;   // 18
static_assert(LOADS_PER_THREAD * 256 * 16 == STAGE_BYTES, "stage must split evenly");
static_assert(MLA_LDS <= 160 * 1024, "LDS budget");

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Hides a value from loop-invariant code motion so per-tile address math is recomputed
// instead of occupying registers across the tile loop.
__device__ __forceinline__ void opaque(int& x) { asm volatile("" : "+v"(x)); }

__global__ __launch_bounds__(256, 1) void sparse_mla_bf16(
    const __bf16* __restrict__ q, const __bf16* __restrict__ kv,
    const int32_t* __restrict__ indices, int k, const int32_t* __restrict__ cu_q,
    const int64_t* __restrict__ cu_k, int nseq, int total_q, int64_t total_k, int H,
    float scale_log2, int nsplit, int rows_per_split, __bf16* __restrict__ out,
    float* __restrict__ lse, float* __restrict__ part_o, float* __restrict__ part_lse) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int split = blockIdx.x;
  const int t = blockIdx.y;
  const int hg = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = lane_id();
  const int half = lane >> 5;
  const int c32 = lane & 31;
  const int rb = wave & 1;        // QK: row block of the tile
  const int hb = wave >> 1;       // QK and PV: head block within the group
  const int dvh = wave & 1;       // PV: value-column half
  const int head_lane = hb * 32 + c32;   // head (within the group) of this lane's softmax stats

  const QueryPos qp = query_pos(cu_q, cu_k, nseq, total_k, t);
  const int64_t L = qp.len;
  const int r_beg = split * rows_per_split;
  const int r_end = min(k, r_beg + rows_per_split);
  const int ntiles = (qp.p >= 0 && L > 0 && r_end > r_beg) ? (r_end - r_beg + TILE - 1) / TILE : 0;
  const int32_t* irow = indices + (int64_t)t * k;
  const __bf16* kvb = kv + qp.key_base * DQK;

  float* xmax = (float*)(lds + OFF_XMAX);     // [2][HG]
  float* xsum = (float*)(lds + OFF_XSUM);     // [2][HG]
  float* xalpha = (float*)(lds + OFF_ALPHA);  // [HG]
  __bf16* pl = (__bf16*)(lds + OFF_P);        // [HG][P_STRIDE]

  f32x16 o[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) o[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  if (ntiles > 0) {
    bf16x8 qreg[36];
    {
      const __bf16* qr = q + ((int64_t)t * H + hg * HG + head_lane) * DQK + half * 8;
#pragma unroll
      for (int st = 0; st < 36; ++st) qreg[st] = *(const bf16x8*)(qr + st * 16);
    }
    auto load_idx = [&](int tile) -> int {
      const int r = r_beg + tile * TILE + lane;
      return (tile < ntiles && r < r_end) ? irow[r] : -1;
    };
    auto issue = [&](int idxv, int stg) {
      char* base = lds + stg * STAGE_BYTES;
      int slot = tid;
      opaque(slot);                          // recomputed per tile instead of held in registers
#pragma unroll
      for (int c = 0; c < LOADS_PER_THREAD; ++c, slot += 256) {
        const int row = slot / CHUNKS;
        const int gc = (slot - row * CHUNKS) ^ (row & 7);
        const int v = __shfl(idxv, row, WAVE);
        const int64_t r = (v >= 0 && v < L) ? v : 0;
        global_to_lds16(kvb + r * DQK + gc * 8, base + (c * 256 + wave * 64) * 16);
      }
    };

    int idx_cur = load_idx(0);
    issue(idx_cur, 0);
    int idx_next = load_idx(1);

    for (int tile = 0; tile < ntiles; ++tile) {
      const int stg = tile & 1;
      wait_all_memory();
      __syncthreads();                       // tile rows landed; previous tile fully consumed
      const int idx_tile = idx_cur;
      if (tile + 1 < ntiles) issue(idx_next, stg ^ 1);
      idx_cur = idx_next;
      idx_next = load_idx(tile + 2);
      const char* sbase = lds + stg * STAGE_BYTES;
      const uint64_t vmask = __ballot(r_beg + tile * TILE + lane < r_end && idx_tile >= 0 &&
                                      idx_tile < L);

      // ---- S^T[32 rows x 32 heads] over the full 576-wide row. Chunk 2*st+half of row arow
      // sits in slot 8*(st/4) + ((2*(st%4)+half) ^ (arow&7)): four lane bases + immediates.
      f32x16 s = {};
      {
        const int arow = rb * 32 + c32;
        const char* abase[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          abase[j] = sbase + arow * ROWB + (((2 * j + half) ^ (arow & 7)) << 4);
#pragma unroll
        for (int st = 0; st < 36; ++st) {
          const bf16x8 a = *(const bf16x8*)(abase[st & 3] + (st >> 2) * 128);
          s = mfma32x32x16(a, qreg[st], s);
        }
      }
      float sv[16];
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = rb * 32 + mfma32_row(r, lane);
        sv[r] = ((vmask >> row) & 1) ? s[r] * scale_log2 : -INFINITY;
        mx = fmaxf(mx, sv[r]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, WAVE));
      if (half == 0) xmax[rb * HG + head_lane] = mx;
      __syncthreads();
      const float m_tile = fmaxf(xmax[head_lane], xmax[HG + head_lane]);
      const float m_new = fmaxf(m_run, m_tile);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = (m_run == -INFINITY) ? 0.f : exp2f(m_run - m_new);
      float ls = 0.f;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p = exp2f(sv[4 * g + e] - m_use);
          ls += p;
          pk[e] = (__bf16)p;
        }
        const int row0 = rb * 32 + 8 * g + 4 * half;
        *(bf16x4*)(pl + head_lane * P_STRIDE + row0) = pk;
      }
      ls += __shfl_xor(ls, 32, WAVE);
      if (half == 0) xsum[rb * HG + head_lane] = ls;
      if (rb == 0 && half == 0) xalpha[head_lane] = alpha;
      __syncthreads();
      l_run = alpha * l_run + xsum[head_lane] + xsum[HG + head_lane];
      m_run = m_new;

      // ---- O[32 heads x 256 cols] = alpha * O + P[32 heads x 64 rows] * V[64 rows x 256 cols]
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float al = xalpha[hb * 32 + mfma32_row(r, lane)];
#pragma unroll
        for (int db = 0; db < 8; ++db) o[db][r] *= al;
      }
      // V[krow][col] for the B operand of value block db, rows 4*rr.. of the lane's k-group:
      // krow & 7 = j16 >> 2 and the chunk of col is 4*(8*dvh + db) + c2, so the swizzled slot is
      // 4*((8*dvh + db) ^ rr) + (c2 ^ (j16 >> 2)): one lane base plus immediate offsets.
      const int g16 = lane >> 4;
      const int j16 = lane & 15;
      const int c2 = 2 * (g16 & 1) + ((j16 & 3) >> 1);
      const char* vbase = sbase + (8 * (g16 >> 1) + (j16 >> 2)) * ROWB +
                          ((c2 ^ (j16 >> 2)) << 4) + (j16 & 1) * 8;
      const __bf16* pbase = pl + head_lane * P_STRIDE + half * 8;
#pragma unroll
      for (int ks = 0; ks < TILE / 16; ++ks) {
        const bf16x8 pa = *(const bf16x8*)(pbase + ks * 16);
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          const int blk0 = 8 * dvh + db;
          const i16x4 v0 = lds_read_tr16(vbase + ks * 16 * ROWB + (blk0 << 6));
          const i16x4 v1 = lds_read_tr16(vbase + ks * 16 * ROWB + 4 * ROWB + ((blk0 ^ 1) << 6));
          const bf16x8 bop = concat_bf16(v0, v1);
          o[db] = mfma32x32x16(pa, bop, o[db]);
        }
      }
    }
  }

  // ---- epilogue: 1/l per head, normalised output (final or partial) and log-sum-exp
  __syncthreads();
  if (rb == 0 && half == 0) {
    xsum[head_lane] = l_run;
    xmax[head_lane] = m_run;
  }
  __syncthreads();
  const int head_base = hg * HG + hb * 32;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int hl = hb * 32 + mfma32_row(r, lane);
    const float l = xsum[hl];
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int64_t h = head_base + mfma32_row(r, lane);
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const int col = dvh * 256 + db * 32 + c32;
      const float v = o[db][r] * inv;
      if (nsplit == 1)
        out[((int64_t)t * H + h) * DV + col] = (__bf16)v;
      else
        part_o[(((int64_t)t * nsplit + split) * H + h) * DV + col] = v;
    }
  }
  if (rb == 0 && dvh == 0 && half == 0) {
    const float l = xsum[head_lane];
    const float val = l > 0.f ? (xmax[head_lane] + log2f(l)) * kLn2 : -INFINITY;
    const int64_t h = hg * HG + head_lane;
    if (nsplit == 1) {
      if (lse) lse[(int64_t)t * H + h] = val;
    } else {
      part_lse[((int64_t)t * nsplit + split) * H + h] = val;
    }
  }
}

// Merge the splits of one (query, head): out = sum_i exp(lse_i - lse) * o_i, lse = logsumexp.
__global__ __launch_bounds__(128) void mla_combine(const float* __restrict__ part_o,
                                                   const float* __restrict__ part_lse,
                                                   int nsplit, int H, __bf16* __restrict__ out,
                                                   float* __restrict__ lse) {
  const int t = blockIdx.x;
  const int h = blockIdx.y;
  const float* pl = part_lse + (int64_t)t * nsplit * H + h;
  float mx = -INFINITY;
  for (int i = 0; i < nsplit; ++i) mx = fmaxf(mx, pl[(int64_t)i * H]);
  float sum = 0.f;
  if (mx != -INFINITY)
    for (int i = 0; i < nsplit; ++i) sum += expf(pl[(int64_t)i * H] - mx);
  const float tot = (mx == -INFINITY) ? -INFINITY : mx + logf(sum);
  f32x4 acc = {};
  const int col = threadIdx.x * 4;
  if (mx != -INFINITY) {
    for (int i = 0; i < nsplit; ++i) {
      const float li = pl[(int64_t)i * H];
      if (li == -INFINITY) continue;
      const float wgt = expf(li - tot);
      const f32x4 v = *(const f32x4*)(part_o + (((int64_t)t * nsplit + i) * H + h) * DV + col);
      acc += wgt * v;
    }
  }
  bf16x4 ob;
#pragma unroll
  for (int e = 0; e < 4; ++e) ob[e] = (__bf16)acc[e];
  *(bf16x4*)(out + ((int64_t)t * H + h) * DV + col) = ob;
  if (lse && threadIdx.x == 0) lse[(int64_t)t * H + h] = tot;
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
  p.workspace = p.nsplit > 1 ? (size_t)b.total_q * p.nsplit * n_heads * (DV + 1) * sizeof(float)
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
  float* part_o = nullptr;
  float* part_lse = nullptr;
  if (plan.nsplit > 1) {
    part_o = (float*)workspace;
    part_lse = part_o + (size_t)b.total_q * plan.nsplit * n_heads * DV;
  }
  dim3 grid(plan.nsplit, b.total_q, n_heads / HG);
  sparse_mla_bf16<<<grid, 256, MLA_LDS, stream>>>(
      (const __bf16*)q, (const __bf16*)kv, indices, k, b.cu_q, b.cu_k, b.nseq, b.total_q,
      b.total_k, n_heads, scale * kLog2e, plan.nsplit, plan.rows_per_split, (__bf16*)out, lse,
      part_o, part_lse);
  e = hipGetLastError();
  if (e != hipSuccess || plan.nsplit == 1) return e;
  mla_combine<<<dim3(b.total_q, n_heads), 128, 0, stream>>>(part_o, part_lse, plan.nsplit,
                                                             n_heads, (__bf16*)out, lse);
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

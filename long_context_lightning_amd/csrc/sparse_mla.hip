// Sparse MLA forward in MQA mode ("How GLM5.3 Sparse Attention Affects HBM Memory Usage",
// How it works / Model): every query head attends, with softmax, over only the top-k selected
// latent rows; the key is the full 576-wide latent+rope row and the value its leading 512
// columns (weight absorption), so one gathered 1152-byte row serves all heads for both products.
//
// bf16 kernel: one workgroup = (query, KV split, group of 64 heads), 8 waves, 160 KB of LDS, one
// workgroup per CU. Waves 0-3 serve heads 0-31 of the group and waves 4-7 heads 32-63; both
// halves compute on the same gathered tile.
//   * Tiles of 64 selected rows are gathered straight from HBM into LDS with direct
//     global->LDS 16-byte loads, double-buffered: the gathers of tile i+1 go out during tile
//     i's QK^T (once the barrier that ended tile i-1, or for tile 0 the one after the query
//     block was read out of stage 1, has freed their stage) and land while
//     tile i computes; at the end of tile i each wave waits for its own gathers and one barrier
//     publishes tile i+1 to the workgroup. Each row's 72 chunks of 16 B are stored with the
//     chunk slot XOR-ed by a 3-bit function of the row (swz) that keeps every MFMA operand read
//     free of LDS bank conflicts.
//   * The first two tiles' indices are loaded before the sequence lookup, so the two latencies
//     overlap at the start of the workgroup; the query block is gathered right behind the
//     first tile. (Gathering it before the lookup was measured: the lookup's memory wait then
//     drains it first and the first tile goes out later, for no gain.)
//   * QK^T is computed transposed, S^T[rows x heads] = KV[rows x 576] * Q^T, on 32x32x16 MFMAs:
//     in each head half, wave (rb, kh) owns rows 32*rb.. and K half kh for all 32 heads; the
//     query half is resident in registers (B operand). The two K-half partial sums of a row
//     block are exchanged through LDS, each wave keeping half of the block's elements, so
//     every lane holds one head.
//   * Softmax in fp32 (base-2 exponent, scale*log2(e) folded into the logits) against a fixed
//     reference maximum per head, raised (with the output block rescaled) only when a logit
//     exceeds it by more than 2^16; P is rounded to bf16 into LDS.
//   * P*V on 32x32x16 MFMAs: wave w of a head half owns value columns 128*w.. of its 32 heads;
//     P is the A operand, V (row-major in the same LDS tile) is read column-wise with the
//     gfx950 transposing LDS read. The fp32 output block stays in registers across tiles.
//   * With several splits per query, each split stores its normalised partial output in bf16,
//     in the accumulator register layout (32 contiguous bytes per lane and value block), and
//     its log-sum-exp; a combine kernel merges them with exp(lse_i - lse) weights. With one
//     split the output block is transposed through LDS and written with 16-byte stores.
//   * Splits: about one workgroup per CU in total (256), but at least two tiles per split (a
//     split's first tile waits out the whole gather latency; its second overlaps it).
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"
#include "select.hpp"

namespace dsa {
namespace {

constexpr int DQK = 576;
constexpr int DV = 512;
constexpr int HG = 32;                       // heads of one head half (one per MFMA column)
constexpr int WG_HEADS = 2 * HG;             // heads per workgroup
constexpr int NWAVES = 8;
constexpr int NTHREADS = NWAVES * WAVE;      // 512
constexpr int TILE = 64;                     // selected rows per LDS stage
constexpr int ROWB = DQK * 2;                // 1152 bytes per latent row
constexpr int CHUNKS = ROWB / 16;            // 72 chunks of 16 B
constexpr int STAGE_BYTES = TILE * ROWB;     // 73728
constexpr int ROPE_OFF = DV * 2;             // byte offset of the RoPE columns in a row
constexpr int XSLOT = 8 * 64 * 4;            // exchange slot of one wave: 8 floats per lane
constexpr int R_BYTES = NWAVES * XSLOT;      // QK exchange, then each wave's P (see below)
constexpr int MLA_LDS = 2 * STAGE_BYTES + R_BYTES;   // 160 KB: one workgroup per CU
constexpr int LOADS_PER_THREAD = STAGE_BYTES / 16 / NTHREADS;   // 9
constexpr int QK_STEPS = DQK / 16 / 2;       // 18 MFMA k-steps per K half
constexpr int VB_WAVE = DV / 32 / 4;         // 4 value blocks of 32 columns per wave
static_assert(LOADS_PER_THREAD * NTHREADS * 16 == STAGE_BYTES, "stage must split evenly");
static_assert(LOADS_PER_THREAD % 3 == 0, "gathers are issued in groups of three");
static_assert(HG * 32 * 2 <= XSLOT, "a wave's P (32 heads x 32 rows) fits one exchange slot");
static_assert(WG_HEADS * DV * 2 <= STAGE_BYTES, "the output block fits one stage");
static_assert(MLA_LDS <= 160 * 1024, "LDS of one CU");

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

// Direct global -> LDS copy of 16 bytes per lane (lane i writes lds_wave_base + 16*i), issued
// as volatile inline assembly that the compiler does not see as a memory access: it then adds
// no waits of its own for these loads (it would wait for all of them before any LDS access,
// since it cannot tell the two stages apart), and the workgroup barriers do not drain them.
// The kernel orders them itself: exact vmcnt waits before a stage is read, and a barrier
// before a stage is refilled (volatile asm is never moved across the barrier's fence).
__device__ __forceinline__ void gather16(const void* gptr, const char* lds_wave_base) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)lds_wave_base);
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(gptr), "{m0}"(m));
}

// Lanes l and l^32 combined (max / sum), in every lane, with one gfx950 lane-half swap: of the
// two results one holds the low half of x in both halves and the other the high half.
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Hides a value from loop-invariant code motion so per-tile address math is recomputed
// instead of occupying registers across the tile loop.
__device__ __forceinline__ void opaque(int& x) { asm volatile("" : "+v"(x)); }

// Softmax statistics live in the RoPE columns of the tile being processed: those columns are
// only read by QK^T, which every wave has finished before the first statistic is written, and
// the prefetch writes the other stage. Float i sits in row i/32 at RoPE byte 4*(i%32).
__device__ __forceinline__ float* stat(char* stage, int i) {
  return (float*)(stage + (i >> 5) * ROWB + ROPE_OFF + (i & 31) * 4);
}
constexpr int ST_MAX = 0;       // [8 waves][HG] maximum over each wave's 16 rows
constexpr int ST_FLAG = 512;    // [8]           wave saw a logit beyond its reference headroom

// Element r of the QK accumulator kept by K-half wave kh after the exchange: value q (0..7) of
// the wave is element 8*(q/4) + 4*kh + q%4; the other eight go to the partner wave.
__device__ __forceinline__ int kept_elem(int q, int kh) { return 8 * (q >> 2) + 4 * kh + (q & 3); }

// ---------------------------------------------------------------------------------------------
// Fused selection (decode rows of at most FUSED_MAX_POS positions): every workgroup of a query
// computes the query's top-k from its score row with the workgroup select of select.hpp (thread
// i holds `per` consecutive positions, 8, 16 or 32 as the row bound needs) and writes only its
// own split's slice of the index row, so the top-k needs no launch of its own. The rule is step
// 2's: the k largest scores among positions 0..p, an equal score going to the lower position,
// every position when p + 1 <= k, ascending.
// ---------------------------------------------------------------------------------------------
constexpr int FUSED_PER = 32;                                 // positions per thread, at most
constexpr int FUSED_MAX_POS = FUSED_PER * NTHREADS;            // 16384
constexpr int SEL_LIST = 2048;                 // longest slice of one split
constexpr int SEL_LIST_AT = sel_scratch_words<NTHREADS>();
constexpr int SEL_SCRATCH_WORDS = SEL_LIST_AT + SEL_LIST;
static_assert(SEL_SCRATCH_WORDS * 4 <= STAGE_BYTES, "fused selection scratch must fit one stage");

// Writes idx_row[r] for r in [r_beg, r_end) (r_end - r_beg <= SEL_LIST) from the scores v of
// positions 0..n-1 (sel_load_scores), and the slice's first 2*TILE entries also to head (LDS;
// entries past the slice are left as they are). scratch: SEL_SCRATCH_WORDS words of LDS whose
// first two histograms and the low-bit summaries were zeroed before a barrier. Every thread of
// the workgroup calls it; a barrier must follow before head is read.
template <int PER>
__device__ __forceinline__ void fused_select_slice(const float (&v)[PER], int64_t n, int k,
                                                   int r_beg, int r_end, int32_t* idx_row,
                                                   uint32_t* __restrict__ scratch,
                                                   int32_t* __restrict__ head) {
  const int tid = threadIdx.x;
  uint32_t* list = scratch + SEL_LIST_AT;      // [SEL_LIST] the split's slice
  if (n <= k) {                                // dense: every visible position
    for (int r = r_beg + tid; r < r_end; r += NTHREADS) {
      const int32_t x = r < n ? r : -1;
      idx_row[r] = x;
      if (r - r_beg < 2 * TILE) head[r - r_beg] = x;
    }
    return;
  }
  uint32_t key[PER];
  sel_keys(v, n, key);
  sel_count0(key, scratch);
  __syncthreads();
  const SelThreshold s = sel_threshold<NTHREADS, PER>(key, (uint32_t)k, scratch);
  typename SelMask<PER>::T m;
  uint32_t rk;
  sel_ranks<NTHREADS, PER>(key, s, scratch + SEL_RED, m, rk);
  // write the taken positions whose ranks fall in [r_beg, r_end), skipping those ranked before
  // r_beg
  uint32_t skip = min((uint32_t)r_beg - min(rk, (uint32_t)r_beg), (uint32_t)sel_popc(m));
  rk += skip;
  while (skip > 0) {
    m &= m - 1;
    --skip;
  }
  while (m != 0 && rk < (uint32_t)r_end) {
    const int i = sel_low_index(m);
    list[rk - r_beg] = (uint32_t)(tid * PER + i);
    m &= m - 1;
    ++rk;
  }
  __syncthreads();
  for (int j = tid; j < r_end - r_beg; j += NTHREADS) {
    idx_row[r_beg + j] = (int32_t)list[j];
    if (j < 2 * TILE) head[j] = (int32_t)list[j];
  }
}

// grid: 1-D, 8 * ceil(T/8) * nsplit * ceil(H/64) workgroups. Consecutive workgroups are
// dispatched round-robin to the 8 XCDs; the mapping gives every workgroup of one query the same
// XCD, so the query block and the split partials of a query stay in one L2, and gives each XCD
// a run of consecutive queries (XCD x: queries x*ceil(T/8) ..), worked through in order, so the
// queries of one sequence (several decode tokens, a prefill chunk) meet in one L2 and the rows
// they select in common are fetched from HBM once.
// FPER > 0: the split's indices are selected from `scores` in the prologue (fused_select_slice,
// FPER positions per thread) and written to `indices` (the caller's index row); the first two
// tiles' indices are taken from LDS, the later ones read back from `indices`.
template <int FPER>
__global__ __launch_bounds__(NTHREADS, 1) void sparse_mla_bf16(
    const __bf16* __restrict__ q, const __bf16* __restrict__ kv,
    const int32_t* __restrict__ indices, int k, const int32_t* __restrict__ cu_q,
    const int64_t* __restrict__ cu_k, int nseq, int total_q, int64_t total_k, int H,
    float scale_log2, int nsplit, int rows_per_split, __bf16* __restrict__ out,
    float* __restrict__ lse, __bf16* __restrict__ part_o, float* __restrict__ part_lse,
    const float* __restrict__ scores, int64_t ld_scores, int32_t* idx_out) {
  constexpr bool FUSED = FPER > 0;
  // Separate LDS objects let the compiler see that the gathers streaming into one stage never
  // alias reads of the other stage or of the exchange region, so it adds no waits of its own.
  __shared__ __attribute__((aligned(16))) char stage0[STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) char stage1[STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) char rbuf[R_BYTES];
  const int nhg = (H + WG_HEADS - 1) / WG_HEADS;
  const int xcd = blockIdx.x & 7;
  const int kk = blockIdx.x >> 3;
  const int hg = kk % nhg;
  const int split = (kk / nhg) % nsplit;
  const int t = xcd * ((total_q + 7) >> 3) + kk / nhg / nsplit;
  if (t >= total_q) return;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = lane_id();
  const int half = lane >> 5;
  const int c32 = lane & 31;
  const int hl = wave >> 2;       // head half of the workgroup
  const int w4 = wave & 3;        // wave within the head half
  const int kh = w4 & 1;          // QK: K half (columns 288*kh ..); softmax: kept element set
  const int rb = w4 >> 1;         // QK: row block (rows 32*rb ..)
  const int cq = w4;              // PV: value columns 128*cq ..
  const int g32 = 2 * hg + hl;    // 32-head group of this head half
  // With H an odd multiple of 32 the upper half of the last group has no heads: it computes on
  // the first group's queries (keeping every wave in step) and writes nothing.
  const bool heads_valid = g32 * HG < H;

  const int r_beg = split * rows_per_split;
  const int r_end = min(k, r_beg + rows_per_split);
  // with FUSED the index row is written by this kernel (idx_out, not restrict-qualified) and
  // read back from it
  const int32_t* irow = (FUSED ? (const int32_t*)idx_out : indices) + (int64_t)t * k;
  // The first two tiles' indices do not depend on the sequence lookup, so their loads go out
  // before it and the latencies overlap. (Loaded even if the split turns out to be empty: every
  // address is inside its array.) The query block is loaded behind the first gathers.
  bf16x8 qreg[QK_STEPS];
  int i_even = 0, i_odd = 0;                            // indices of the next even / odd tile
  if constexpr (!FUSED) {
    i_even = irow[min(r_beg + lane, k - 1)];
    i_odd = irow[min(r_beg + TILE + lane, k - 1)];
  }
  // The sequence lookup is done by one wave and shared through LDS: every workgroup of the grid
  // starts at once and reads the same few cache lines of cu_seqlens.
  float fs[FUSED ? FPER : 1];                           // this thread's scores (FUSED)
  if constexpr (FUSED)                                  // issued before the sequence lookup
    sel_load_scores<FPER>(scores + (int64_t)t * ld_scores,
                            min(ld_scores, (int64_t)FUSED_MAX_POS), (ld_scores & 3) == 0, fs);
  if constexpr (FUSED) sel_clear<NTHREADS>((uint32_t*)stage0, 3);   // (ordered by the lookup's barrier)
  QueryPos qp;
  {
    int64_t* qs = (int64_t*)rbuf;
    if (wave == 0) {
      const QueryPos q0 = query_pos(cu_q, cu_k, nseq, total_k, t);
      if (lane == 0) {
        qs[0] = q0.p;
        qs[1] = q0.key_base;
        qs[2] = q0.len;
      }
    }
    __syncthreads();
    qp.p = qs[0];
    qp.key_base = qs[1];
    qp.len = qs[2];
    qp.b = 0;
  }
  if constexpr (FUSED) {
    // this split's slice of the index row, then the first two tiles' indices read back (the
    // barrier's workgroup fence orders the stores before the loads)
    const int64_t n = qp.p >= 0 ? min(min(qp.p + 1, ld_scores), (int64_t)FUSED_MAX_POS) : 0;
    int32_t* head = (int32_t*)rbuf + 64;      // past the lookup's words
    fused_select_slice<FPER>(fs, n, k, r_beg, r_end, idx_out + (int64_t)t * k, (uint32_t*)stage0,
                             head);
    __syncthreads();
    // entries past the slice are masked before use
    i_even = head[lane];
    i_odd = head[TILE + lane];
  }
  const int64_t L = qp.len;
  const uint32_t Lu = (uint32_t)min(L, (int64_t)0x7fffffff);
  const int ntiles = (qp.p >= 0 && L > 0 && r_end > r_beg) ? (r_end - r_beg + TILE - 1) / TILE : 0;
  const __bf16* kvb = kv + qp.key_base * DQK;
  // QK exchange: wave w writes slot w and reads slot w^1, which no other wave reads. Once its
  // reads have returned, wave w reuses slot w^1 for its probabilities: [2][32 heads][8 rows]
  // bf16 (row group g of its 16 rows per head; lane half h holds rows 4h..4h+3 of a group), so
  // no wave writes a slot that another wave may still be reading.
  float* xch = (float*)rbuf;                  // [8 waves][2][64 lanes][4]

  // Softmax with a fixed reference maximum per head: the first tile in which a head has a finite
  // logit sets its reference m_ref, and probabilities are exp2(s - m_ref) without rescaling the
  // output block. Only if a later tile exceeds a reference by more than 2^kHeadroom is it raised,
  // with the head's output block and running sum scaled by exp2(old - new) (online softmax).
  f32x16 o[VB_WAVE];
  float l_part = 0.f;             // this wave's share (its rows) of the softmax sum of head c32
  // reference maxima of head c32 in both head halves: every wave tracks both and updates them
  // from the same shared statistics, so every decision on them is uniform across the workgroup
  float mref0 = -INFINITY, mref1 = -INFINITY;
  {                                           // 0 x 0 + 0 on the matrix core keeps o in AGPRs
    const bf16x8 z = {};
#pragma unroll
    for (int db = 0; db < VB_WAVE; ++db) o[db] = mfma32x32x16(z, z, f32x16{});
  }

  if (ntiles > 0) {
    // Index of tile row `lane` as loaded: the load is issued for every tile number, clamped into
    // the row, so that each tile costs the same number of memory operations. Rows past the split
    // are masked where the index is used (a select right after the load would wait for it).
    auto load_idx = [&](int tile) __attribute__((always_inline)) -> int {
      return irow[min(r_beg + tile * TILE + lane, k - 1)];
    };
    auto masked = [&](int tile, int v) __attribute__((always_inline)) -> int {
      return (tile < ntiles && r_beg + tile * TILE + lane < r_end) ? v : -1;
    };
    // gathers one tile into stage `stg`: slot c*512+tid holds chunk (slot%72)^swz(row) of row
    // slot/72 (invalid rows read row 0 and are masked later)
    auto issue = [&](char* stg, int tile, int idx_raw) __attribute__((always_inline)) {
      const int idxv = masked(tile, idx_raw);
      int tt = tid;
      opaque(tt);
#pragma unroll
      for (int g = 0; g < LOADS_PER_THREAD / 3; ++g) {
        int vs[3], gcs[3];
#pragma unroll
        for (int j = 0; j < 3; ++j) {
          // the 64 slots of this wave lie in rows r0 and r0+1 (72 slots per row): two scalar
          // reads of the index register instead of a cross-lane shuffle
          const int sbase = (g * 3 + j) * NTHREADS + wave * 64;      // wave-uniform
          const int r0 = sbase / CHUNKS;
          const int slot = (g * 3 + j) * NTHREADS + tt;
          const int row = slot / CHUNKS;
          gcs[j] = (slot - row * CHUNKS) ^ swz(row);
          const int i0 = __builtin_amdgcn_readlane(idxv, r0);
          const int i1 = __builtin_amdgcn_readlane(idxv, min(r0 + 1, TILE - 1));
          vs[j] = row == r0 ? i0 : i1;
        }
#pragma unroll
        for (int j = 0; j < 3; ++j) {
          const uint32_t v = (uint32_t)vs[j] < Lu ? (uint32_t)vs[j] : 0u;
          gather16(kvb + (size_t)v * DQK + gcs[j] * 8, stg + ((g * 3 + j) * NTHREADS + wave * 64) * 16);
        }
        __builtin_amdgcn_sched_barrier(0);   // keep the groups apart: bounded live registers
      }
    };
    // gather number jj (of LOADS_PER_THREAD) of a tile into stage `stg`, for the index vi of
    // the tile row this lane's slot lies in (fetched beforehand with one cross-lane read)
    auto issue_one = [&](char* stg, int vi, int jj) __attribute__((always_inline)) {
      const int sbase = jj * NTHREADS + wave * 64;                     // wave-uniform
      const int slot = jj * NTHREADS + tid;
      const int row = slot / CHUNKS;
      const int gc = (slot - row * CHUNKS) ^ swz(row);
      const uint32_t v = (uint32_t)vi < Lu ? (uint32_t)vi : 0u;
      gather16(kvb + (size_t)v * DQK + gc * 8, stg + sbase * 16);
    };
    // Double buffering: tile j computes in stage j%2 while the gathers of tile j+1 stream into
    // the other stage. The indices of tile j+2 are loaded at the top of tile j (into the
    // register that held tile j's). At the end of tile j each wave waits for all its memory
    // operations (the gathers of tile j+1 have had a whole tile of compute to land), and one
    // barrier then both frees stage j and publishes tile j+1; the gathers of tile j+2 follow.
    // row-validity masks of the next even / odd tile, taken right after a full wait (so the
    // compiler never has to wait for an index load at the top of a tile)
    uint64_t vm_even = 0, vm_odd = 0;
    {
      wait_all_memory();
      vm_even = __ballot((uint32_t)masked(0, i_even) < Lu);
      vm_odd = __ballot((uint32_t)masked(1, i_odd) < Lu);
      // The query block [64 heads x 576] has the shape of a tile: it is gathered the same way,
      // coalesced, into stage 1 (the upper half of the last group of an odd number of 32-head
      // groups reads heads 0..31 again), and each wave reads its B operands from there with
      // the same conflict-free pattern as the QK A operands. It goes out first and tile 0
      // right behind it; loads complete in issue order, so the query block is read into
      // registers while tile 0 still streams in.
      {
        int tt = tid;
        opaque(tt);
        const __bf16* qt = q + (int64_t)t * H * DQK;
#pragma unroll
        for (int j = 0; j < LOADS_PER_THREAD; ++j) {
          const int slot = j * NTHREADS + tt;
          const int row = slot / CHUNKS;
          const int head = hg * WG_HEADS + row < H ? hg * WG_HEADS + row : (row & (HG - 1));
          gather16(qt + (int64_t)head * DQK + ((slot - row * CHUNKS) ^ swz(row)) * 8,
                   stage1 + (j * NTHREADS + wave * 64) * 16);
        }
      }
      issue(stage0, 0, i_even);
      wait_vmcnt<LOADS_PER_THREAD>();          // this wave's query-block gathers
      __syncthreads();                         // every wave's
      {
        const int row = hl * HG + c32;
        const int sq = swz(row);
#pragma unroll
        for (int i = 0; i < QK_STEPS; ++i) {
          const int chunk = 36 * kh + 2 * i + half;
          qreg[i] = *(const bf16x8*)(stage1 + row * ROWB + ((chunk ^ sq) << 4));
        }
        // in registers before stage 1 is refilled (and before any use in the loop)
#pragma unroll
        for (int i = 0; i < QK_STEPS; ++i) asm volatile("" : "+v"(qreg[i]));
      }
      __syncthreads();
      // Tile 1 goes out during tile 0's QK^T like every later tile, not here: issued behind
      // tile 0 it shares the HBM queue with it and delays the first tile, and its stage could
      // not take tile 2 before tile 0 ends anyway (measured: 2-5% faster per call).
      wait_all_memory();
      __syncthreads();                         // tile 0 published
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

    auto tile_max = [&](char* stage, int h) __attribute__((always_inline)) -> float {
      return fmaxf(fmaxf(*stat(stage, ST_MAX + (4 * h + 0) * HG + c32), *stat(stage, ST_MAX + (4 * h + 1) * HG + c32)),
                   fmaxf(*stat(stage, ST_MAX + (4 * h + 2) * HG + c32), *stat(stage, ST_MAX + (4 * h + 3) * HG + c32)));
    };
    // Tile maxima through LDS (every wave's row maxima, one barrier): unset references are set;
    // a reference exceeded by more than the headroom is raised to the tile maximum, and the
    // output block and running sum of its head are scaled by exp2(old - new) (online softmax;
    // rare, so the common path keeps every accumulator update on the matrix core).
    auto update_refs = [&](char* stage, float mx) __attribute__((always_inline)) {
      if (half == 0) *stat(stage, ST_MAX + wave * HG + c32) = mx;
      __syncthreads();
      const float mt0 = tile_max(stage, 0), mt1 = tile_max(stage, 1);
      const bool r0 = mref0 != -INFINITY && mt0 > mref0 + kHeadroom;
      const bool r1 = mref1 != -INFINITY && mt1 > mref1 + kHeadroom;
      const float f0 = r0 ? __builtin_amdgcn_exp2f(mref0 - mt0) : 1.f;
      const float f1 = r1 ? __builtin_amdgcn_exp2f(mref1 - mt1) : 1.f;
      if (mref0 == -INFINITY || r0) mref0 = mt0;
      if (mref1 == -INFINITY || r1) mref1 = mt1;
      if (__ballot(r0 || r1) != 0) {           // uniform across the workgroup
        // every value a lane holds belongs to its own head (hl, c32)
        const float f = hl ? f1 : f0;
#pragma unroll
        for (int r = 0; r < 16; ++r)
#pragma unroll
          for (int db = 0; db < VB_WAVE; ++db) o[db][r] *= f;
        l_part *= f;
      }
    };
    // probabilities exp2(s - m_ref) of this wave's 16 rows for head c32 into P (bf16); returns
    // their sum
    auto write_p = [&](const float (&sv)[8]) __attribute__((always_inline)) -> float {
      const float m_ref = hl ? mref1 : mref0;
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
        // rows 32*rb + 16*g + 8*kh + 4*half + e of head c32
        *(bf16x4*)(rbuf + (wave ^ 1) * XSLOT + (g * HG + c32) * 16 + half * 8) = pk;
      }
      return halves_sum(ls);
    };

    // One tile in stage `stage`; idx holds the indices of this tile and receives those of
    // tile+2, vm the row-validity mask of this tile and then of tile+2. The gathers of tile+1
    // (into `other`, freed by the barrier that ended the previous tile) are issued here,
    // spread over the QK^T steps, so their address arithmetic hides behind the matrix core;
    // idx_next holds tile+1's indices.
    auto step = [&](char* stage, char* other, int tile, int& idx, uint64_t& vm, int idx_next)
        __attribute__((always_inline)) {
      const uint64_t vmask = vm;
      idx = load_idx(tile + 2);

      // ---- QK^T half sums: S^T[32 rows x 32 heads] over this wave's 288 columns
      f32x16 s = {};
      {
        bf16x8 a[2];
        auto rd = [&](int i, int b) __attribute__((always_inline)) { a[b] = *(const bf16x8*)(stage + abase[i & 3] + (i >> 2) * 128); };
        static_assert(2 * LOADS_PER_THREAD == QK_STEPS, "one gather per two QK steps");
        rd(0, 0);
        if (tile + 1 < ntiles) {    // uniform
          const int idxv = masked(tile + 1, idx_next);
          // the index of each gather's tile row, read across lanes (lane r holds row r's)
          int vsel[LOADS_PER_THREAD];
#pragma unroll
          for (int jj = 0; jj < LOADS_PER_THREAD; ++jj)
            vsel[jj] = __builtin_amdgcn_ds_bpermute(((jj * NTHREADS + tid) / CHUNKS) * 4, idxv);
#pragma unroll
          for (int i = 0; i < QK_STEPS; ++i) {
            if (i + 1 < QK_STEPS) rd(i + 1, (i + 1) & 1);
            s = mfma32x32x16(a[i & 1], qreg[i], s);
            if ((i & 1) == 0) issue_one(other, vsel[i >> 1], i >> 1);
          }
        } else {
#pragma unroll
          for (int i = 0; i < QK_STEPS; ++i) {
            if (i + 1 < QK_STEPS) rd(i + 1, (i + 1) & 1);
            s = mfma32x32x16(a[i & 1], qreg[i], s);
          }
        }
      }
      // ---- exchange half sums: keep element set kh, hand the other to the partner wave
      // kh is wave-uniform; both candidate elements are read at compile-time positions and made
      // opaque (an empty asm, no instruction) so the selects are not folded back into an indexed
      // register move
      // The eight handed-over values of a lane go out as two 16-byte writes ([wave][half][lane]
      // layout: each write is 64 lanes x 16 contiguous bytes, free of bank conflicts).
      float e0[8], e1[8];
      f32x4 give[2];
#pragma unroll
      for (int qi = 0; qi < 8; ++qi) {
        e0[qi] = s[kept_elem(qi, 0)];
        e1[qi] = s[kept_elem(qi, 1)];
        asm volatile("" : "+v"(e0[qi]), "+v"(e1[qi]));
        give[qi >> 2][qi & 3] = kh ? e0[qi] : e1[qi];
      }
      f32x4* xch4 = reinterpret_cast<f32x4*>(xch);
      xch4[(wave * 2 + 0) * 64 + lane] = give[0];
      xch4[(wave * 2 + 1) * 64 + lane] = give[1];
      __syncthreads();
      f32x4 part[2];
      part[0] = xch4[((wave ^ 1) * 2 + 0) * 64 + lane];
      part[1] = xch4[((wave ^ 1) * 2 + 1) * 64 + lane];
      // Kept element qi of this lane is row r0 + 16*(qi/4) + qi%4 of the tile, r0 = 32*rb + 8*kh
      // + 4*half: all eight validity bits come from one shift of the tile's mask.
      const uint32_t vbits = (uint32_t)(vmask >> (32 * rb + 8 * kh + 4 * half));
      float sv[8];
      float mx = -INFINITY;
#pragma unroll
      for (int qi = 0; qi < 8; ++qi) {
        const float mine = kh ? e1[qi] : e0[qi];
        sv[qi] = (mine + part[qi >> 2][qi & 3]) * scale_log2;
      }
      if (__builtin_expect(vmask != ~0ull, 0)) {   // uniform: some row of the tile is invalid
#pragma unroll
        for (int qi = 0; qi < 8; ++qi)
          sv[qi] = ((vbits >> (16 * (qi >> 2) + (qi & 3))) & 1) ? sv[qi] : -INFINITY;
      }
#pragma unroll
      for (int qi = 0; qi < 8; ++qi) mx = fmaxf(mx, sv[qi]);
      mx = halves_max(mx);                     // this wave's 16 rows, head c32 of its half
      // The tile maxima are exchanged only while some reference is unset; afterwards a logit
      // beyond its reference's headroom is detected from the wave's own rows and flagged with
      // the probabilities.
      const bool need_max = __ballot(mref0 == -INFINITY || mref1 == -INFINITY) != 0;
      if (need_max) update_refs(stage, mx);
      float ls = write_p(sv);
      const float m_ref = hl ? mref1 : mref0;
      const bool exceed = !need_max && mx > m_ref + kHeadroom;
      const bool wave_exceeds = __ballot(exceed) != 0;   // ballot with every lane active
      if (lane == 0) *stat(stage, ST_FLAG + wave) = wave_exceeds ? 1.f : 0.f;
      __syncthreads();
      float flags = 0.f;
#pragma unroll
      for (int w = 0; w < NWAVES; ++w) flags += *stat(stage, ST_FLAG + w);
      if (flags != 0.f) {                      // uniform: raise, rescale, redo the probabilities
        update_refs(stage, mx);
        ls = write_p(sv);
        __syncthreads();
      }
      l_part += ls;

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
        // P rows 16*ks + 8*half .. +7 of head c32 were written by wave (hl, rb = ks/2, kh = half)
        // into slot 4*hl + 2*(ks/2) + (half^1), row group ks%2
        const char* pbase = rbuf + (4 * hl + (half ^ 1)) * XSLOT + c32 * 16;
#pragma unroll
        for (int ks = 0; ks < TILE / 16; ++ks) {
          const bf16x8 pa = *(const bf16x8*)(pbase + (ks >> 1) * 2 * XSLOT + (ks & 1) * HG * 16);
#pragma unroll
          for (int db = 0; db < VB_WAVE; ++db) {
            const int blk = VB_WAVE * cq + db;
            const i16x4 v0 = lds_read_tr16(vb[0][db & 1] + ks * 16 * ROWB + (blk << 6));
            const i16x4 v1 = lds_read_tr16(vb[1][db & 1] + ks * 16 * ROWB + (blk << 6));
            o[db] = mfma32x32x16(concat_bf16(v0, v1), pa, o[db]);
          }
        }
      }
      // end of the tile: this wave's memory operations (the next tile's gathers and the index
      // load) complete, then one barrier frees this stage and P and publishes the next tile.
      // (Unconditional, also after the last tile: the compiler then knows every index load is
      // complete before the next tile and adds no wait of its own, which would also drain the
      // gathers it cannot see.)
      wait_all_memory();
      vm = __ballot((uint32_t)masked(tile + 2, idx) < Lu);
      __syncthreads();
    };
    for (int tile = 0; tile < ntiles; tile += 2) {   // unrolled by two: each step names its stage
      step(stage0, stage1, tile, i_even, vm_even, i_odd);
      if (tile + 1 < ntiles) step(stage1, stage0, tile + 1, i_odd, vm_odd, i_even);
    }
    wait_all_memory();
  }

  // ---- epilogue: 1/l per head, normalised output (final or partial) and log-sum-exp
  // fin [w4][64 heads]: each wave's share of the softmax sum per head; every lane then adds the
  // four shares of its own head. After the tiles no barrier is needed before fin is written (the
  // last tile's barrier ended every read of rbuf); without tiles the sequence lookup's reads of
  // rbuf are still to be ordered.
  float* fin = (float*)rbuf;
  if (ntiles == 0) __syncthreads();
  if (half == 0) fin[w4 * WG_HEADS + hl * HG + c32] = l_part;
  __syncthreads();
  const int hh = hl * HG + c32;
  const float l_sum =
      (fin[hh] + fin[WG_HEADS + hh]) + (fin[2 * WG_HEADS + hh] + fin[3 * WG_HEADS + hh]);
  // Every value a lane holds belongs to head (hl, c32): element r of value block db is column
  // 32*(VB_WAVE*cq + db) + 8*(r/4) + 4*half + r%4, so each group of four elements is four
  // consecutive columns of the head's output row. The normalised [64 heads x 512] block is
  // staged in LDS as 8-byte pieces (rows padded to OT_PITCH bytes, so the 32 heads of a store
  // fall on distinct bank pairs), then written with 16-byte stores, each wave instruction 1 KB
  // of one row: the final output with one split, else this split's partial output (the same
  // row-major layout, one block per split), which the merge kernel streams back.
  {
    constexpr int OT_PITCH = DV * 2 + 16;
    static_assert(WG_HEADS * OT_PITCH <= STAGE_BYTES, "the staged block fits one stage");
    const float l = l_sum;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    char* orow_lds = stage0 + (hl * HG + c32) * OT_PITCH + (VB_WAVE * cq * 32 + 4 * half) * 2;
#pragma unroll
    for (int db = 0; db < VB_WAVE; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (__bf16)(o[db][4 * g + e] * inv);
        *(bf16x4*)(orow_lds + (db * 32 + 8 * g) * 2) = v;
      }
    __syncthreads();
    __bf16* ob = (nsplit == 1 ? out + (int64_t)t * H * DV
                              : part_o + ((int64_t)t * nsplit + split) * H * DV) +
                 (int64_t)hg * WG_HEADS * DV;
    const int pieces = min(WG_HEADS, H - hg * WG_HEADS) * (DV / 8);
    // Non-temporal stores: the block is read by the next launch (the merge, or the caller), and
    // lines left dirty in L2 would have to be written back at the end of this launch before the
    // next one may start (decode call 29.2 -> 28.0 us with the partials stored this way).
    for (int piece = tid; piece < pieces; piece += NTHREADS) {
      const int row = piece >> 6, c = piece & 63;
      __builtin_nontemporal_store(*(const bf16x8*)(stage0 + row * OT_PITCH + c * 16),
                                  (bf16x8*)(ob + piece * 8));
    }
  }
  if (w4 == 0 && half == 0 && heads_valid) {
    // the reference maxima are uniform across the workgroup
    const float l = l_sum;
    const float val = l > 0.f ? ((hl ? mref1 : mref0) + log2f(l)) * kLn2 : -INFINITY;
    const int64_t h = g32 * HG + c32;
    if (nsplit == 1) {
      if (lse) lse[(int64_t)t * H + h] = val;
    } else {
      part_lse[((int64_t)t * nsplit + split) * H + h] = val;
    }
  }
}

// Merges the splits of every (query, head): out = sum_i exp(lse_i - lse) * o_i with
// lse = logsumexp_i lse_i (natural-log units), o_i the normalised partial outputs. P adjacent
// threads share one piece of 8 consecutive output columns (64 pieces per head); thread p takes
// splits p, p+P, .. (at most CMB_SPLITS of them) and issues all their partial and log-sum-exp
// loads at once, so a merge is one memory round trip; maxima, sums and the weighted partial sums
// then meet across the P threads with lane exchanges. A query's merge runs on the XCD whose L2
// its split partials went through (IndexShare's 8-query layers: 18.3 -> 16.6 us per call).
constexpr int CMB_THREADS = 256;
constexpr int CMB_SPLITS = 8;

template <int P>
__global__ __launch_bounds__(CMB_THREADS) void mla_combine(const __bf16* __restrict__ part_o,
                                                           const float* __restrict__ part_lse,
                                                           int nsplit, int H, int total_q,
                                                           int xrun, __bf16* __restrict__ out,
                                                           float* __restrict__ lse) {
  // xrun > 0: the workgroups of query t run on the XCD whose workgroups of the main kernel made
  // its partials (queries in runs of xrun per XCD, as there); else in plain order
  int64_t blk = blockIdx.x;
  if (xrun > 0) {
    const int64_t per_q = (int64_t)H * 64 * P / CMB_THREADS;     // workgroups of one query
    const int64_t kk = blockIdx.x >> 3;
    blk = ((int64_t)(blockIdx.x & 7) * xrun + kk / per_q) * per_q + kk % per_q;
  }
  const int64_t gid = blk * CMB_THREADS + threadIdx.x;
  const int p = (int)(gid & (P - 1));
  const int64_t piece = gid / P;
  const int c8 = (int)(piece & 63);            // columns 8*c8 .. 8*c8+7
  const int64_t th = piece >> 6;               // t * H + h
  if (th >= (int64_t)total_q * H) return;      // all P threads of a piece together
  const int64_t t = th / H;
  const int64_t h = th - t * H;
  const float* pl = part_lse + t * nsplit * H + h;                 // split i at pl[i * H]
  const __bf16* po = part_o + (t * nsplit * H + h) * DV + c8 * 8;  // split i at po[i * H * DV]
  bf16x8 v[CMB_SPLITS];
  float li[CMB_SPLITS];
#pragma unroll
  for (int j = 0; j < CMB_SPLITS; ++j) {       // past the last split: a clamped copy, unused
    const int i = min(p + j * P, nsplit - 1);
    v[j] = *(const bf16x8*)(po + (int64_t)i * H * DV);
    li[j] = pl[(int64_t)i * H];
  }
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < CMB_SPLITS; ++j)
    if (p + j * P < nsplit) m = fmaxf(m, li[j]);
#pragma unroll
  for (int o = 1; o < P; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, WAVE));
  const float m2 = m * kLog2e;
  float e[CMB_SPLITS], sum = 0.f;
#pragma unroll
  for (int j = 0; j < CMB_SPLITS; ++j) {
    e[j] = (p + j * P < nsplit && li[j] != -INFINITY) ? __builtin_amdgcn_exp2f(li[j] * kLog2e - m2)
                                                       : 0.f;
    sum += e[j];
  }
#pragma unroll
  for (int o = 1; o < P; o <<= 1) sum += __shfl_xor(sum, o, WAVE);
  // sum >= 1 when m is finite (the maximal split contributes exp2(0))
  const float inv = m != -INFINITY ? 1.f / sum : 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < CMB_SPLITS; ++j)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = fmaf(e[j], (float)v[j][c], acc[c]);
#pragma unroll
  for (int o = 1; o < P; o <<= 1)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] += __shfl_xor(acc[c], o, WAVE);
  if (p == 0) {
    bf16x8 r;
#pragma unroll
    for (int c = 0; c < 8; ++c) r[c] = (__bf16)(acc[c] * inv);
    __builtin_nontemporal_store(r, (bf16x8*)(out + th * DV + c8 * 8));   // see the main kernel
    if (lse && c8 == 0)
      lse[th] = m == -INFINITY ? -INFINITY : (m2 + __builtin_amdgcn_logf(sum)) * kLn2;
  }
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

bool fused_select_supported(const Batch& b, const MlaPlan& plan) {
  return b.max_k <= FUSED_MAX_POS && plan.rows_per_split <= SEL_LIST;
}

MlaPlan plan_sparse_mla_bf16(const Batch& b, int k, int n_heads) {
  MlaPlan p;
  const int tiles = (k + TILE - 1) / TILE;
  const int64_t wgs = (int64_t)b.total_q * ((n_heads + WG_HEADS - 1) / WG_HEADS);
  const int64_t wgs1 = wgs > 0 ? wgs : 1;
  int nsplit = (int)((256 + wgs1 - 1) / wgs1);          // one workgroup per CU
  // at least two tiles per split: a split's first tile waits out the whole gather latency, its
  // second tile's gathers overlap the first's compute, and every split adds a partial to merge
  nsplit = std::max(1, std::min(nsplit, (tiles + 1) / 2));
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
                                  hipStream_t stream, const float* fused_scores,
                                  int64_t ld_scores) {
  float* part_lse = nullptr;
  __bf16* part_o = nullptr;
  if (plan.nsplit > 1) {
    part_lse = (float*)workspace;
    part_o = (__bf16*)(part_lse + (size_t)b.total_q * plan.nsplit * n_heads);
  }
  const int tgroups = (b.total_q + 7) / 8;
  const int64_t nblocks =
      (int64_t)8 * tgroups * plan.nsplit * ((n_heads + WG_HEADS - 1) / WG_HEADS);
  auto run = [&](auto kern, const float* sc, int64_t ld, int32_t* idx_out) {
    kern<<<dim3((unsigned)nblocks), NTHREADS, 0, stream>>>(
        (const __bf16*)q, (const __bf16*)kv, indices, k, b.cu_q, b.cu_k, b.nseq, b.total_q,
        b.total_k, n_heads, scale * kLog2e, plan.nsplit, plan.rows_per_split, (__bf16*)out, lse,
        part_o, part_lse, sc, ld, idx_out);
  };
  if (fused_scores) {
    // positions per thread: the fewest that cover the row bound
    const int64_t lim = std::min<int64_t>(ld_scores, FUSED_MAX_POS);
    int32_t* idx_out = const_cast<int32_t*>(indices);
    if (lim <= 8 * NTHREADS) run(sparse_mla_bf16<8>, fused_scores, ld_scores, idx_out);
    else if (lim <= 16 * NTHREADS) run(sparse_mla_bf16<16>, fused_scores, ld_scores, idx_out);
    else run(sparse_mla_bf16<32>, fused_scores, ld_scores, idx_out);
  } else {
    run(sparse_mla_bf16<0>, nullptr, 0, nullptr);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.nsplit == 1) return e;
  // P threads per 8-column piece, each merging at most CMB_SPLITS splits
  int P = 1;
  while (P * CMB_SPLITS < plan.nsplit) P *= 2;
  const int64_t cthreads = (int64_t)b.total_q * n_heads * (DV / 8) * P;
  // XCD runs as in the main kernel when a query's threads fill whole workgroups (then the grid
  // is 8 * ceil(T/8) runs of whole queries; workgroups past total_q leave at once)
  const bool whole = ((int64_t)n_heads * 64 * P) % CMB_THREADS == 0;
  const int64_t per_q = (int64_t)n_heads * 64 * P / CMB_THREADS;
  const int xrun = whole ? tgroups : 0;
  const dim3 cgrid((unsigned)(whole ? 8 * tgroups * per_q
                                    : (cthreads + CMB_THREADS - 1) / CMB_THREADS));
  auto cmb = [&](auto kern) {
    kern<<<cgrid, CMB_THREADS, 0, stream>>>(part_o, part_lse, plan.nsplit, n_heads, b.total_q,
                                            xrun, (__bf16*)out, lse);
  };
  switch (P) {
    case 1: cmb(mla_combine<1>); break;
    case 2: cmb(mla_combine<2>); break;
    case 4: cmb(mla_combine<4>); break;
    case 8: cmb(mla_combine<8>); break;
    case 16: cmb(mla_combine<16>); break;
    case 32: cmb(mla_combine<32>); break;
    default: cmb(mla_combine<64>); break;
  }
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

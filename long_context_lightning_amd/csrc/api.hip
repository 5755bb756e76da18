// C ABI of libdsa: host-side validation, workspace layout and launch sequencing.
// Every check runs before anything is enqueued; calls only enqueue work on the caller's stream.
#include <algorithm>
#include <cmath>
#include <mutex>
#include <vector>

#include "../../include/dsa.h"
#include "kernels.hpp"

using dsa::Batch;

// Scratch of dsa_sparse_mla_fwd_noalloc (the split partials of the sparse-MLA kernel), one copy
// per GPU, held until the process ends. In host code this name stands for the symbol, not for a
// device address: the address on each GPU comes from hipGetSymbolAddress (noalloc_scratch()).
static __device__ __align__(256) char dsa_noalloc_scratch[DSA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of dsa_noalloc_scratch, per device

// Device address of the scratch array on the device of `stream`, looked up once per device with
// that device current.
hipError_t noalloc_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(dsa_noalloc_scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool batch_ok(const dsa_batch* b) {
  return b && b->batch >= 1 && b->total_q >= 0 && b->total_k >= 0 && b->max_seqlen_q >= 1 &&
         b->max_seqlen_k >= 1 && b->cu_seqlens_q && b->cu_seqlens_k &&
         (int64_t)b->max_seqlen_q <= (int64_t)b->max_seqlen_k &&
         b->total_k <= (int64_t)b->batch * b->max_seqlen_k &&
         (int64_t)b->total_q <= (int64_t)b->batch * b->max_seqlen_q &&
         b->total_q <= b->total_k;
}

Batch to_batch(const dsa_batch* b) {
  Batch r;
  r.nseq = b->batch;
  r.total_q = b->total_q;
  r.total_k = b->total_k;
  r.max_q = b->max_seqlen_q;
  r.max_k = b->max_seqlen_k;
  r.cu_q = b->cu_seqlens_q;
  r.cu_k = b->cu_seqlens_k;
  return r;
}

dsa_status from_hip(hipError_t e) { return e == hipSuccess ? DSA_OK : DSA_ERR_HIP; }

// Indexer inputs; the score buffer is checked by the caller.
dsa_status check_indexer(const dsa_batch* b, const void* q_idx, const void* k_idx, const float* w,
                         int32_t hi, int32_t di, dsa_dtype dt, int64_t ld) {
  if (!batch_ok(b) || !q_idx || !k_idx || !w || hi <= 0 || di <= 0 || ld < b->max_seqlen_k)
    return DSA_ERR_INVALID_ARG;
  if (dt == DSA_BF16 || dt == DSA_FP8_E4M3) {
    if (di != 128 || (hi != 32 && hi != 64)) return DSA_ERR_UNSUPPORTED;
  } else if (dt == DSA_F32) {
    if (di > 256 || hi > 128) return DSA_ERR_UNSUPPORTED;
  } else {
    return DSA_ERR_INVALID_ARG;
  }
  return DSA_OK;
}

dsa_status check_mla(const dsa_batch* b, const void* q, const void* kv, const int32_t* indices,
                     int32_t k, int32_t h, int32_t dqk, int32_t dv, float scale, dsa_dtype dt,
                     const void* out) {
  if (!batch_ok(b) || !q || !kv || !indices || !out || k <= 0 || h <= 0 || dqk <= 0 ||
      dv <= 0 || dv > dqk || !std::isfinite(scale))
    return DSA_ERR_INVALID_ARG;
  if (dt == DSA_BF16) {
    if (dqk != 576 || dv != 512 || h % 32 != 0) return DSA_ERR_UNSUPPORTED;
  } else if (dt == DSA_F32) {
    if (dqk > 1024 || h > 1024 || k > dsa::kMaxF32TopK) return DSA_ERR_UNSUPPORTED;
  } else {
    return DSA_ERR_INVALID_ARG;
  }
  return DSA_OK;
}

size_t mla_ws(const dsa_batch* b, int32_t k, int32_t h, dsa_dtype dt) {
  if (dt != DSA_BF16) return 0;
  return dsa::plan_sparse_mla_bf16(to_batch(b), k, h).workspace;
}

size_t scores_bytes(const dsa_batch* b) {
  return align_up((size_t)b->total_q * (size_t)b->max_seqlen_k * sizeof(float));
}

// Selection scratch of the fused call: enough for the per-position top-k and for the block
// selection of any block size (the smallest, 4, needs the most).
size_t select_bytes(const Batch& b, int32_t k) {
  return align_up(std::max(dsa::topk_workspace_bytes(b, k), dsa::block_topk_workspace_bytes(b, 4)));
}

// The launches of dsa_indexer_scores / dsa_indexer_scores_fp8 / dsa_topk after their argument
// checks. The decode indexer kernels also zero-fill `zero` on the side (then *zeroed is true),
// which lets the one-launch split top-k of the same step skip its own zero-fill launch.
dsa_status run_indexer(const dsa_batch* batch, const void* q_idx, const void* k_idx,
                       const float* k_scale, const float* w, int32_t index_n_heads,
                       int32_t index_head_dim, dsa_dtype dtype, float* scores, int64_t ld,
                       hipStream_t stream, dsa::ZeroFill zero = {}, bool* zeroed = nullptr) {
  if (zeroed) *zeroed = false;
  if (batch->total_q == 0 || batch->total_k == 0) return DSA_OK;
  const Batch b = to_batch(batch);
  if (dtype == DSA_FP8_E4M3)
    return from_hip(dsa::launch_indexer_fp8(b, q_idx, k_idx, k_scale, w, index_n_heads, scores,
                                            ld, stream, zero, zeroed));
  if (dtype == DSA_BF16)
    return from_hip(dsa::launch_indexer_bf16(b, q_idx, k_idx, w, index_n_heads, scores, ld,
                                             stream, zero, zeroed));
  return from_hip(dsa::launch_indexer_f32(b, (const float*)q_idx, (const float*)k_idx, w,
                                          index_n_heads, index_head_dim, scores, ld, stream));
}

}  // namespace

extern "C" {

dsa_status dsa_indexer_scores(const dsa_batch* batch, const void* q_idx, const void* k_idx,
                              const float* w, int32_t index_n_heads, int32_t index_head_dim,
                              dsa_dtype dtype, float* scores, int64_t ld_scores,
                              hipStream_t stream) {
  if (!scores) return DSA_ERR_INVALID_ARG;
  if (dtype == DSA_FP8_E4M3) return DSA_ERR_UNSUPPORTED;   // dsa_indexer_scores_fp8
  dsa_status st = check_indexer(batch, q_idx, k_idx, w, index_n_heads, index_head_dim, dtype,
                                ld_scores);
  if (st != DSA_OK) return st;
  return run_indexer(batch, q_idx, k_idx, nullptr, w, index_n_heads, index_head_dim, dtype,
                     scores, ld_scores, stream);
}

dsa_status dsa_indexer_scores_fp8(const dsa_batch* batch, const void* q_idx, const void* k_idx,
                                  const float* k_scale, const float* w, int32_t index_n_heads,
                                  int32_t index_head_dim, float* scores, int64_t ld_scores,
                                  hipStream_t stream) {
  if (!scores) return DSA_ERR_INVALID_ARG;
  dsa_status st = check_indexer(batch, q_idx, k_idx, w, index_n_heads, index_head_dim,
                                DSA_FP8_E4M3, ld_scores);
  if (st != DSA_OK) return st;
  return run_indexer(batch, q_idx, k_idx, k_scale, w, index_n_heads, index_head_dim,
                     DSA_FP8_E4M3, scores, ld_scores, stream);
}

dsa_status dsa_topk(const dsa_batch* batch, const float* scores, int64_t ld_scores,
                    int32_t index_topk, int32_t* indices, void* workspace, size_t ws_bytes,
                    hipStream_t stream) {
  if (!batch_ok(batch) || !scores || !indices || index_topk <= 0 ||
      ld_scores < batch->max_seqlen_k)
    return DSA_ERR_INVALID_ARG;
  const Batch b = to_batch(batch);
  const size_t need = dsa::topk_workspace_bytes(b, index_topk);
  if (need > 0 && (!workspace || ws_bytes < need)) return DSA_ERR_WORKSPACE;
  if (batch->total_q == 0) return DSA_OK;
  return from_hip(dsa::launch_topk(b, scores, ld_scores, index_topk, indices, workspace, stream));
}

dsa_status dsa_block_topk(const dsa_batch* batch, const float* scores, int64_t ld_scores,
                          int32_t block_size, dsa_pool pool, int32_t topk_blocks,
                          int32_t* indices, void* workspace, size_t ws_bytes,
                          hipStream_t stream) {
  if (!batch_ok(batch) || !scores || !indices || topk_blocks <= 0 || block_size <= 0 ||
      ld_scores < batch->max_seqlen_k || (pool != DSA_POOL_MAX && pool != DSA_POOL_MEAN))
    return DSA_ERR_INVALID_ARG;
  const Batch b = to_batch(batch);
  if (!dsa::block_topk_supported(b, block_size, topk_blocks)) return DSA_ERR_UNSUPPORTED;
  const size_t need = dsa::block_topk_workspace_bytes(b, block_size);
  if (need > 0 && (!workspace || ws_bytes < need)) return DSA_ERR_WORKSPACE;
  if (batch->total_q == 0) return DSA_OK;
  return from_hip(dsa::launch_block_topk(b, scores, ld_scores, block_size, pool == DSA_POOL_MEAN,
                                         topk_blocks, indices, workspace, stream));
}

size_t dsa_block_topk_workspace_size(const dsa_batch* batch, int32_t block_size) {
  if (!batch_ok(batch) || block_size <= 0) return 0;
  return dsa::block_topk_workspace_bytes(to_batch(batch), block_size);
}

dsa_status dsa_sparse_mla_fwd(const dsa_batch* batch, const void* q, const void* kv,
                              const int32_t* indices, int32_t index_topk, int32_t n_heads,
                              int32_t d_qk, int32_t d_v, float softmax_scale, dsa_dtype dtype,
                              void* out, float* lse, void* workspace, size_t ws_bytes,
                              hipStream_t stream) {
  dsa_status st = check_mla(batch, q, kv, indices, index_topk, n_heads, d_qk, d_v,
                            softmax_scale, dtype, out);
  if (st != DSA_OK) return st;
  const Batch b = to_batch(batch);
  if (dtype == DSA_BF16) {
    const dsa::MlaPlan plan = dsa::plan_sparse_mla_bf16(b, index_topk, n_heads);
    if (plan.workspace > 0 && (!workspace || ws_bytes < plan.workspace)) return DSA_ERR_WORKSPACE;
    if (batch->total_q == 0) return DSA_OK;
    return from_hip(dsa::launch_sparse_mla_bf16(b, q, kv, indices, index_topk, n_heads,
                                                softmax_scale, out, lse, workspace, plan,
                                                stream));
  }
  if (batch->total_q == 0) return DSA_OK;
  return from_hip(dsa::launch_sparse_mla_f32(b, (const float*)q, (const float*)kv, indices,
                                             index_topk, n_heads, d_qk, d_v, softmax_scale,
                                             (float*)out, lse, stream));
}

dsa_status dsa_sparse_mla_fwd_noalloc(const dsa_batch* batch, const void* q, const void* kv,
                                      const int32_t* indices, int32_t index_topk,
                                      int32_t n_heads, int32_t d_qk, int32_t d_v,
                                      float softmax_scale, dsa_dtype dtype, void* out, float* lse,
                                      hipStream_t stream) {
  dsa_status st = check_mla(batch, q, kv, indices, index_topk, n_heads, d_qk, d_v,
                            softmax_scale, dtype, out);
  if (st != DSA_OK) return st;
  if (dtype != DSA_BF16)     // the fp32 kernel uses no scratch
    return dsa_sparse_mla_fwd(batch, q, kv, indices, index_topk, n_heads, d_qk, d_v,
                              softmax_scale, dtype, out, lse, nullptr, 0, stream);
  const Batch b = to_batch(batch);
  const dsa::MlaPlan plan = dsa::plan_sparse_mla_bf16(b, index_topk, n_heads);
  if (plan.workspace > DSA_NOALLOC_SCRATCH_BYTES) return DSA_ERR_WORKSPACE;
  if (batch->total_q == 0) return DSA_OK;
  void* scratch = nullptr;
  if (plan.workspace > 0) {
    const hipError_t e = noalloc_scratch(stream, &scratch);
    if (e != hipSuccess) return DSA_ERR_HIP;
  }
  return from_hip(dsa::launch_sparse_mla_bf16(b, q, kv, indices, index_topk, n_heads,
                                              softmax_scale, out, lse, scratch, plan, stream));
}

size_t dsa_workspace_size(dsa_op op, const dsa_batch* batch, int32_t index_topk,
                          int32_t n_heads, int32_t d_v) {
  if (!batch_ok(batch) || index_topk <= 0) return 0;
  const Batch b = to_batch(batch);
  // only the bf16 (d_v = 512) sparse-MLA kernel splits the selected rows and needs scratch
  const bool split_kv = n_heads > 0 && n_heads % 32 == 0 && d_v == 512;
  const size_t mla = split_kv ? mla_ws(batch, index_topk, n_heads, DSA_BF16) : 0;
  switch (op) {
    case DSA_OP_INDEXER:
      return 0;
    case DSA_OP_TOPK:
      return dsa::topk_workspace_bytes(b, index_topk);
    case DSA_OP_SPARSE_MLA:
      return mla;
    case DSA_OP_FORWARD:
      return scores_bytes(batch) + select_bytes(b, index_topk) + align_up(mla);
  }
  return 0;
}

dsa_status dsa_forward(const dsa_batch* batch, const dsa_forward_args* a, int32_t* shared_indices,
                       int32_t compute_indices, void* out, float* lse, void* workspace,
                       size_t ws_bytes, hipStream_t stream) {
  if (!a || !shared_indices || (compute_indices != 0 && compute_indices != 1) ||
      (a->index_fp8 != 0 && a->index_fp8 != 1) || a->block_size < 0 ||
      (a->block_size > 0 && (a->index_topk % a->block_size != 0 ||
                             (a->pool != DSA_POOL_MAX && a->pool != DSA_POOL_MEAN))))
    return DSA_ERR_INVALID_ARG;
  const dsa_dtype idx_dt = a->index_fp8 ? DSA_FP8_E4M3 : a->dtype;
  dsa_status st = check_mla(batch, a->q, a->kv, shared_indices, a->index_topk, a->n_heads,
                            a->d_qk, a->d_v, a->softmax_scale, a->dtype, out);
  if (st != DSA_OK) return st;
  const Batch b = to_batch(batch);
  const size_t s_bytes = compute_indices ? scores_bytes(batch) : 0;
  const size_t t_bytes = compute_indices ? select_bytes(b, a->index_topk) : 0;
  const size_t m_bytes = mla_ws(batch, a->index_topk, a->n_heads, a->dtype);
  const size_t need = s_bytes + t_bytes + m_bytes;
  if (need > 0 && (!workspace || ws_bytes < need)) return DSA_ERR_WORKSPACE;
  char* ws = (char*)workspace;
  float* scores = (float*)ws;
  const int64_t ld = batch->max_seqlen_k;
  if (compute_indices) {
    st = check_indexer(batch, a->q_idx, a->k_idx, a->w, a->index_n_heads, a->index_head_dim,
                       idx_dt, ld);
    if (st != DSA_OK) return st;
  }
  if (batch->total_q == 0) return DSA_OK;
  if (compute_indices) {
    const dsa::MlaPlan fplan = dsa::plan_sparse_mla_bf16(b, a->index_topk, a->n_heads);
    const bool fused =
        a->block_size == 0 && a->dtype == DSA_BF16 && dsa::fused_select_supported(b, fplan);
    // the one-launch split top-k needs its row state zero: the decode indexer clears it on the
    // side, so the top-k needs no zero-fill launch of its own
    dsa::ZeroFill zero;
    if (!fused && a->block_size == 0 && ((uintptr_t)(ws + s_bytes) & 15) == 0) {
      zero.words = dsa::topk_state_words(b, a->index_topk);
      zero.p = zero.words > 0 ? (uint32_t*)(ws + s_bytes) : nullptr;
    }
    bool zeroed = false;
    st = run_indexer(batch, a->q_idx, a->k_idx, a->index_fp8 ? a->k_idx_scale : nullptr, a->w,
                     a->index_n_heads, a->index_head_dim, idx_dt, scores, ld, stream, zero,
                     &zeroed);
    if (st != DSA_OK) return st;
    if (fused) {
      // rows of at most 16384 positions: the sparse-MLA kernel selects each query's top-k in its
      // prologue (one launch fewer); it writes shared_indices as dsa_topk would
      return from_hip(dsa::launch_sparse_mla_bf16(b, a->q, a->kv, shared_indices, a->index_topk,
                                                  a->n_heads, a->softmax_scale, out, lse,
                                                  ws + s_bytes + t_bytes, fplan, stream, scores,
                                                  ld));
    }
    st = a->block_size > 0
             ? dsa_block_topk(batch, scores, ld, a->block_size, (dsa_pool)a->pool,
                              a->index_topk / a->block_size, shared_indices, ws + s_bytes,
                              t_bytes, stream)
             : from_hip(dsa::launch_topk(b, scores, ld, a->index_topk, shared_indices,
                                         ws + s_bytes, stream, zeroed));
    if (st != DSA_OK) return st;
  }
  return dsa_sparse_mla_fwd(batch, a->q, a->kv, shared_indices, a->index_topk, a->n_heads,
                            a->d_qk, a->d_v, a->softmax_scale, a->dtype, out, lse,
                            ws + s_bytes + t_bytes, m_bytes, stream);
}

dsa_status dsa_check_batch(const dsa_batch* batch, hipStream_t stream) {
  if (!batch_ok(batch)) return DSA_ERR_INVALID_ARG;
  const int B = batch->batch;
  std::vector<int32_t> cq(B + 1);
  std::vector<int64_t> ck(B + 1);
  if (hipStreamSynchronize(stream) != hipSuccess) return DSA_ERR_HIP;
  if (hipMemcpy(cq.data(), batch->cu_seqlens_q, (B + 1) * sizeof(int32_t),
                hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(ck.data(), batch->cu_seqlens_k, (B + 1) * sizeof(int64_t),
                hipMemcpyDeviceToHost) != hipSuccess)
    return DSA_ERR_HIP;
  if (cq[0] != 0 || ck[0] != 0 || cq[B] != batch->total_q || ck[B] != batch->total_k)
    return DSA_ERR_BATCH;
  for (int b = 0; b < B; ++b) {
    const int64_t nq = (int64_t)cq[b + 1] - cq[b];
    const int64_t L = ck[b + 1] - ck[b];
    if (nq < 1 || L < nq || nq > batch->max_seqlen_q || L > batch->max_seqlen_k)
      return DSA_ERR_BATCH;
  }
  return DSA_OK;
}

const char* dsa_status_string(dsa_status s) {
  switch (s) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_INVALID_ARG: return "DSA_ERR_INVALID_ARG: invalid argument";
    case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED: shape or dtype not compiled";
    case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE: workspace missing or too small";
    case DSA_ERR_HIP: return "DSA_ERR_HIP: HIP runtime error";
    case DSA_ERR_BATCH: return "DSA_ERR_BATCH: cu_seqlens inconsistent with batch sizes";
  }
  return "unknown dsa_status";
}

int32_t dsa_version(void) { return 200; }

}  // extern "C"

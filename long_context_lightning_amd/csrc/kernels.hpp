// Host-side launch interface of the libdsa kernels (one translation unit per step).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

struct Batch {
  int nseq;
  int total_q;
  int64_t total_k;
  int max_q;
  int max_k;
  const int32_t* cu_q;
  const int64_t* cu_k;
};

// Words a launch zero-fills on the side (the next step's state), or none.
struct ZeroFill {
  uint32_t* p = nullptr;
  int64_t words = 0;
};

// Step 1: lightning indexer. index_head_dim is 128 on the bf16 path. The decode kernels also
// zero-fill `zero` (and then return true in *zeroed); the prefill kernel does not.
hipError_t launch_indexer_bf16(const Batch& b, const void* q_idx, const void* k_idx,
                               const float* w, int index_n_heads, float* scores, int64_t ld,
                               hipStream_t stream, ZeroFill zero = {}, bool* zeroed = nullptr);
// fp8 (e4m3fn) queries and keys; k_scale [total_k] or null.
hipError_t launch_indexer_fp8(const Batch& b, const void* q_idx, const void* k_idx,
                              const float* k_scale, const float* w, int index_n_heads,
                              float* scores, int64_t ld, hipStream_t stream, ZeroFill zero = {},
                              bool* zeroed = nullptr);
hipError_t launch_indexer_f32(const Batch& b, const float* q_idx, const float* k_idx,
                              const float* w, int index_n_heads, int index_head_dim,
                              float* scores, int64_t ld, hipStream_t stream);

// Step 2: causal top-k.
size_t topk_workspace_bytes(const Batch& b, int k);
// Words at the start of the top-k workspace that must be zero when the top-k starts (the row
// state of the one-launch split path), or 0. launch_topk zero-fills them with a launch of its
// own unless state_zeroed says an earlier launch on the stream already has.
int64_t topk_state_words(const Batch& b, int k);
hipError_t launch_topk(const Batch& b, const float* scores, int64_t ld, int k, int32_t* indices,
                       void* workspace, hipStream_t stream, bool state_zeroed = false);

// Step 2, block-pooled: blocks of `block` positions scored by their max (or mean) score, the kb
// best blocks' positions written to indices [T, kb * block]; workspace: block keys.
bool block_topk_supported(const Batch& b, int block, int kb);
size_t block_topk_workspace_bytes(const Batch& b, int block);
hipError_t launch_block_topk(const Batch& b, const float* scores, int64_t ld, int block,
                             bool mean, int kb, int32_t* indices, void* workspace,
                             hipStream_t stream);

// Step 3: sparse MLA (MQA) forward.
struct MlaPlan {
  int nsplit;
  int rows_per_split;
  size_t workspace;
};
MlaPlan plan_sparse_mla_bf16(const Batch& b, int k, int n_heads);
// With fused_scores, the top-k selection of each query runs in the kernel's prologue from the
// score rows [T, ld_scores] and `indices` (then written, [T, k]) receives it; rows of at most
// 16384 positions and splits of at most 2048 indices (fused_select_supported).
bool fused_select_supported(const Batch& b, const MlaPlan& plan);
hipError_t launch_sparse_mla_bf16(const Batch& b, const void* q, const void* kv,
                                  const int32_t* indices, int k, int n_heads, float scale,
                                  void* out, float* lse, void* workspace, const MlaPlan& plan,
                                  hipStream_t stream, const float* fused_scores = nullptr,
                                  int64_t ld_scores = 0);
hipError_t launch_sparse_mla_f32(const Batch& b, const float* q, const float* kv,
                                 const int32_t* indices, int k, int n_heads, int d_qk, int d_v,
                                 float scale, float* out, float* lse, hipStream_t stream);

constexpr int kMaxF32TopK = 8192;  // fp32 path keeps one softmax row in LDS

}  // namespace dsa

/*
 * libdsa — DeepSeek Sparse Attention (DSA) hot path for AMD Instinct MI355X (gfx950).
 *
 * The path has three steps, as the pages describe them:
 *   1. lightning indexer: every past token of a query gets a score, the per-head weighted sum
 *      of ReLU(query-head . key) over the indexer heads, one key row per token
 *      ("How GLM5.3 Sparse Attention Affects HBM Memory Usage", How it works / Model;
 *      "DeepSeek Sparse Attention" technique page, In the code: ReLU(q.k) weighted sums);
 *   2. per-query causal top-k (index_topk = 2048; below k visible tokens attention stays dense),
 *      one selection shared by all attention heads (same page and section);
 *   3. sparse MLA in MQA mode: every query head attends with softmax over only the selected
 *      latent rows; the key is the whole latent+rope row, the value its leading d_v columns
 *      (same page and section; the 120.8 FLOP/B decode intensity at 64 heads fixes this layout).
 *   IndexShare (same page, How it works / IndexShare): one indexer + top-k pass serves a group
 *   of layers; its cached indices are reused by the other layers of the group.
 *
 * Conventions shared by every call
 *   - Ragged batch (dsa_batch): sequence b owns query rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1
 *     and key / latent rows cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1; L_b = its context length.
 *     Query j of sequence b (nq_b new queries, nq_b <= L_b) sits at position p = L_b - nq_b + j
 *     and sees sequence positions 0..p (itself included).
 *   - All tensors are dense row-major device buffers owned by the caller. The library never
 *     allocates, frees or synchronises on a call path; each call only enqueues work on `stream`
 *     and returns. Scratch memory comes from a caller-provided workspace whose size is given by
 *     dsa_workspace_size(). Mutable global state: (1) one write-only device array of the
 *     prefill indexer: lanes with no score to store (causally masked keys, keys or queries past
 *     a sequence) store into it, so every key tile issues the same number of stores; it is
 *     never read, so concurrent calls on several streams store into it without affecting any
 *     result; (2) the scratch array of dsa_sparse_mla_fwd_noalloc (see there), used by that
 *     call only.
 *   - All argument checks run on the host before anything is enqueued; a non-zero status means
 *     nothing was launched. Device-resident values (cu_seqlens) cannot be checked without a
 *     synchronisation: the caller guarantees they are consistent with the host-side sizes, and
 *     every kernel clamps its reads to total_q / total_k / ld so inconsistent values give wrong
 *     results, never out-of-bounds accesses. dsa_check_batch() validates them on demand (it
 *     synchronises the stream).
 *   - A failed kernel launch returns DSA_ERR_HIP; the HIP error stays readable through
 *     hipGetLastError().
 *   - Supported shapes: bf16 with (d_qk, d_v, index_head_dim) = (576, 512, 128),
 *     n_heads a multiple of 32, index_n_heads 32 or 64; fp32 with d_qk <= 1024, d_v <= d_qk,
 *     index_head_dim <= 256, n_heads <= 1024, index_n_heads <= 128. Other combinations return
 *     DSA_ERR_UNSUPPORTED.
 */
#ifndef LIBDSA_DSA_H
#define LIBDSA_DSA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = 1,   /* null pointer, negative size, inconsistent sizes            */
  DSA_ERR_UNSUPPORTED = 2,   /* valid but not compiled: dims / dtype combination           */
  DSA_ERR_WORKSPACE = 3,     /* workspace null or smaller than dsa_workspace_size()        */
  DSA_ERR_HIP = 4,           /* a HIP runtime call or kernel launch failed                 */
  DSA_ERR_BATCH = 5          /* dsa_check_batch(): cu_seqlens inconsistent with the sizes  */
} dsa_status;

/* Element types. DSA_FP8_E4M3 is OCP fp8 e4m3fn (1 byte; finite values up to 448, no infinity),
 * accepted for the indexer inputs q_idx / k_idx only (dsa_indexer_scores_fp8, and dsa_forward
 * with index_fp8 = 1). */
typedef enum { DSA_F32 = 0, DSA_BF16 = 1, DSA_FP8_E4M3 = 2 } dsa_dtype;

/* Ragged batch description. Host integers plus two device arrays. */
typedef struct {
  int32_t batch;                 /* B >= 1                                                    */
  int32_t total_q;               /* T = rows of q, q_idx, w, out, lse, indices, scores        */
  int64_t total_k;               /* rows of kv and k_idx = cu_seqlens_k[B]                     */
  int32_t max_seqlen_q;          /* max_b nq_b (>= 1)                                          */
  int32_t max_seqlen_k;          /* max_b L_b (>= 1); row length bound for scores             */
  const int32_t* cu_seqlens_q;   /* device [B+1], cu_seqlens_q[0] = 0, cu_seqlens_q[B] = T     */
  const int64_t* cu_seqlens_k;   /* device [B+1], cu_seqlens_k[0] = 0, cu_seqlens_k[B] = total_k */
} dsa_batch;

/* Step 1 — lightning indexer ("How GLM5.3 Sparse Attention Affects HBM Memory Usage",
 * How it works / Model).
 *   scores[t * ld_scores + s] = sum_j w[t, j] * max(0, sum_c q_idx[t, j, c] * k_idx[cu_k[b] + s, c])
 * for every query t (of sequence b, position p) and s = 0..p. Entries s > p are not written.
 *   q_idx  [T, index_n_heads, index_head_dim]  dtype
 *   k_idx  [total_k, index_head_dim]           dtype (one key row per token, shared by heads)
 *   w      [T, index_n_heads]                  fp32
 *   scores [T, ld_scores]                      fp32, ld_scores >= max_seqlen_k
 * Products are accumulated in fp32; integer-valued inputs whose sums stay below 2^24 give
 * exact scores. q_idx, k_idx and w must be finite: the bf16 kernels are compiled without NaN
 * semantics (the ReLU is a plain maximum), so a NaN or infinite input gives unspecified scores. */
dsa_status dsa_indexer_scores(const dsa_batch* batch, const void* q_idx, const void* k_idx,
                              const float* w, int32_t index_n_heads, int32_t index_head_dim,
                              dsa_dtype dtype, float* scores, int64_t ld_scores,
                              hipStream_t stream);

/* Step 1 with fp8 indexer inputs ("How GLM5.3 Sparse Attention Affects HBM Memory Usage",
 * Evidence: the serving stacks run the decode path in FP8; "Sparse attention" glossary page,
 * Why it matters: precision support decides the realised speed-up). q_idx and k_idx hold OCP
 * e4m3fn bytes with the layouts above (index_head_dim = 128, index_n_heads 32 or 64); k_scale
 * [total_k] fp32 is one non-negative scale per key row, or NULL for 1. The score is step 1's
 * formula on the dequantised keys k_idx[s] * k_scale[s]:
 *   scores[t * ld_scores + s] = k_scale[s] * sum_j w[t, j] * max(0, q_idx[t, j, :] . k_idx[s, :])
 * (equal because max(0, c x) = c max(0, x) for c >= 0). Per-(token, head) query scales, if any,
 * are non-negative factors of the same kind and go into w. Products are exact and accumulated in
 * fp32, so integer-valued inputs with sums below 2^24 and power-of-two scales give exact scores.
 * NaN bytes (0x7f, 0xff) in q_idx / k_idx give unspecified scores. */
dsa_status dsa_indexer_scores_fp8(const dsa_batch* batch, const void* q_idx, const void* k_idx,
                                  const float* k_scale, const float* w, int32_t index_n_heads,
                                  int32_t index_head_dim, float* scores, int64_t ld_scores,
                                  hipStream_t stream);

/* Step 2 — causal top-k (same page and section: top-k 2048, dense below k).
 * For query t at position p: if p + 1 <= index_topk, indices[t] = 0, 1, .., p, then -1;
 * otherwise the index_topk positions with the largest scores among 0..p, where scores compare
 * as real numbers (-0.0 == +0.0) and an equal score goes to the lower position. The selected
 * positions are written in ascending order.
 *   scores  [T, ld_scores] fp32 (only s <= p is read)
 *   indices [T, index_topk] int32, sequence-local positions
 *   workspace: dsa_workspace_size(DSA_OP_TOPK, ...) bytes (may be 0 bytes / NULL when that is 0).
 *     It is non-zero for batches of at most 64 query rows whose longest sequence exceeds 32768
 *     keys: those rows are split over several workgroups that meet through per-row histograms
 *     and counts kept there. Its contents on entry do not matter (the call zero-fills what it
 *     needs); on return they are undefined. For rows of at most 2,097,152 positions, whose
 *     workgroups the device can hold at once (its compute units times the kernel's occupancy,
 *     queried once per device), the row's workgroups meet at barriers inside one launch
 *     (device-scope counters, polled): such a
 *     barrier waits for workgroups of the same row only, which are dispatched before any later
 *     row's, so it always completes once they can run; its polls are bounded (about a second),
 *     so if other work kept a row's workgroups from running that long the launch still ends,
 *     with that row's indices undefined. Longer rows take five launches.
 * Scores must not be NaN. */
dsa_status dsa_topk(const dsa_batch* batch, const float* scores, int64_t ld_scores,
                    int32_t index_topk, int32_t* indices, void* workspace, size_t ws_bytes,
                    hipStream_t stream);

/* Step 2, block-pooled variant ("DeepSeek Sparse Attention" technique page, In the code:
 * MiniMax-M3 pools its indexer scores into blocks and keeps the top index_topk_blocks blocks per
 * query; GLM-5.3-Flash scores pooled candidates).
 * For query t at position p, positions 0..p are cut into blocks of block_size consecutive
 * positions (the last block holds the remainder). A block's score is the maximum (DSA_POOL_MAX)
 * or the mean over its visible positions (DSA_POOL_MEAN, an fp32 quotient) of its scores. The
 * topk_blocks best blocks are chosen as step 2 chooses positions (scores compare as reals, an
 * equal score goes to the lower block; every block when at most topk_blocks are visible), and
 * indices[t] lists every visible position of the chosen blocks, ascending, padded with -1:
 *   scores  [T, ld_scores] fp32 (only s <= p is read; must not be NaN)
 *   indices [T, topk_blocks * block_size] int32, sequence-local positions; pass
 *           index_topk = topk_blocks * block_size to the sparse-MLA call that reads them.
 * block_size is a power of two in 4..256, 1 <= topk_blocks <= 1024, and max_seqlen_k /
 * block_size (rounded up) at most 32768; otherwise DSA_ERR_UNSUPPORTED.
 * workspace: dsa_block_topk_workspace_size() bytes (the block scores); contents on entry do not
 * matter, on return they are undefined. Mean pooling sums in fp32: for integer-valued scores
 * whose block sums stay below 2^24 the block scores are exact quotients. */
typedef enum { DSA_POOL_MAX = 0, DSA_POOL_MEAN = 1 } dsa_pool;
dsa_status dsa_block_topk(const dsa_batch* batch, const float* scores, int64_t ld_scores,
                          int32_t block_size, dsa_pool pool, int32_t topk_blocks,
                          int32_t* indices, void* workspace, size_t ws_bytes,
                          hipStream_t stream);
size_t dsa_block_topk_workspace_size(const dsa_batch* batch, int32_t block_size);

/* Step 3 — sparse MLA forward in MQA mode (same page and section).
 *   z_s = softmax_scale * sum_{c < d_qk} q[t, h, c] * kv[cu_k[b] + s, c]   for s in indices[t]
 *   out[t, h, :] = sum_s softmax(z)_s * kv[cu_k[b] + s, 0:d_v];  lse[t, h] = ln sum_s exp(z_s)
 *   q       [T, n_heads, d_qk]   dtype
 *   kv      [total_k, d_qk]      dtype (latent + rope row; its first d_v columns are the value)
 *   indices [T, index_topk]      int32 sequence-local positions in any order; entries < 0 are
 *                                skipped; entries >= L_b are skipped; duplicates count twice.
 *   out     [T, n_heads, d_v]    dtype;  lse [T, n_heads] fp32 or NULL.
 * softmax_scale must be finite (DSA_ERR_INVALID_ARG otherwise).
 * A query with no valid index gets out = 0 and lse = -inf. Softmax statistics and the output
 * accumulator are fp32; probabilities are rounded to bf16 for the value product on the bf16
 * path.
 *   workspace: dsa_workspace_size(DSA_OP_SPARSE_MLA, ...) bytes (may be NULL when that is 0).
 *     When a query's selected rows are split over several workgroups (few queries, bf16), it
 *     holds each split's normalised partial output (bf16) and log-sum-exp, merged by a second
 *     kernel. Its contents on entry do not matter; on return they are undefined. */
dsa_status dsa_sparse_mla_fwd(const dsa_batch* batch, const void* q, const void* kv,
                              const int32_t* indices, int32_t index_topk, int32_t n_heads,
                              int32_t d_qk, int32_t d_v, float softmax_scale, dsa_dtype dtype,
                              void* out, float* lse, void* workspace, size_t ws_bytes,
                              hipStream_t stream);

/* Step 3 without a workspace argument, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). Arguments,
 * results and status codes are those of dsa_sparse_mla_fwd; the scratch that call keeps in the
 * caller's workspace (each split's partial output and log-sum-exp) lives instead in a
 * library-owned device array of DSA_NOALLOC_SCRATCH_BYTES on each GPU, which the GPU holds
 * until the process ends. Nothing is allocated or freed. A call that would need more scratch
 * than that (dsa_workspace_size(DSA_OP_SPARSE_MLA, ...) bytes) returns DSA_ERR_WORKSPACE with
 * nothing enqueued. Every call on one GPU uses the same array and nothing in it needs to start
 * at zero: calls ordered on one stream are safe, calls that overlap in time on one GPU (several
 * streams or threads) race and give wrong results. The first call on a GPU looks the array's
 * device address up (hipGetSymbolAddress, with that GPU current); make it before any graph
 * capture that records this call. */
#define DSA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
dsa_status dsa_sparse_mla_fwd_noalloc(const dsa_batch* batch, const void* q, const void* kv,
                                      const int32_t* indices, int32_t index_topk,
                                      int32_t n_heads, int32_t d_qk, int32_t d_v,
                                      float softmax_scale, dsa_dtype dtype, void* out, float* lse,
                                      hipStream_t stream);

/* Inputs of the three steps, for the fused call. */
typedef struct {
  const void* q_idx;             /* [T, index_n_heads, index_head_dim]                         */
  const void* k_idx;             /* [total_k, index_head_dim]                                  */
  const float* w;                /* [T, index_n_heads]                                         */
  int32_t index_n_heads;
  int32_t index_head_dim;
  int32_t index_topk;
  const void* q;                 /* [T, n_heads, d_qk]                                         */
  const void* kv;                /* [total_k, d_qk]                                            */
  int32_t n_heads;
  int32_t d_qk;
  int32_t d_v;
  float softmax_scale;
  dsa_dtype dtype;               /* q, kv, out; and q_idx, k_idx unless index_fp8             */
  int32_t index_fp8;             /* 1: q_idx, k_idx are fp8 e4m3fn (dsa_indexer_scores_fp8)     */
  const float* k_idx_scale;      /* with index_fp8: [total_k] key scales, or NULL for 1        */
  int32_t block_size;            /* 0: step 2 per position; else block-pooled selection        */
                                 /* (dsa_block_topk) of index_topk / block_size blocks          */
  int32_t pool;                  /* with block_size: DSA_POOL_MAX or DSA_POOL_MEAN             */
} dsa_forward_args;

/* Whole path with IndexShare (same page, How it works / IndexShare).
 * compute_indices = 1: indexer + top-k write shared_indices [T, index_topk], then sparse MLA
 *                      reads them (q_idx, k_idx, w must be valid).
 * compute_indices = 0: shared_indices is read as cached by an earlier call of the group;
 *                      q_idx / k_idx / w are ignored and may be NULL.
 * With block_size > 0 the selection is dsa_block_topk's (index_topk a multiple of block_size).
 * Per-position selection on the bf16 path with max_seqlen_k <= 16384 runs inside the sparse-MLA
 * launch (each attention workgroup selects its own slice of shared_indices from the score row),
 * so the top-k takes no launch of its own; shared_indices and the outputs are the same as with
 * the separate calls, bit for bit. When the top-k splits long rows over workgroups in one launch
 * (see dsa_topk), the decode indexer launch zero-fills that launch's row state on the side, so
 * the top-k is one launch here too.
 * The workspace holds the [T, max_seqlen_k] fp32 score matrix plus the selection and split-KV
 * scratch: dsa_workspace_size(DSA_OP_FORWARD, ...) bytes (enough for either selection). */
dsa_status dsa_forward(const dsa_batch* batch, const dsa_forward_args* args,
                       int32_t* shared_indices, int32_t compute_indices, void* out, float* lse,
                       void* workspace, size_t ws_bytes, hipStream_t stream);

typedef enum {
  DSA_OP_INDEXER = 0,            /* needs no workspace                                         */
  DSA_OP_TOPK = 1,
  DSA_OP_SPARSE_MLA = 2,
  DSA_OP_FORWARD = 3
} dsa_op;

/* Workspace bytes needed by `op` for this batch (host sizes only). 0 on invalid arguments. */
size_t dsa_workspace_size(dsa_op op, const dsa_batch* batch, int32_t index_topk,
                          int32_t n_heads, int32_t d_v);

/* Copies cu_seqlens to the host (synchronising `stream`) and checks them against the host
 * sizes: monotone, cu_q[0] = cu_k[0] = 0, cu_q[B] = total_q, cu_k[B] = total_k,
 * 1 <= nq_b <= L_b, max_b nq_b <= max_seqlen_q, max_b L_b <= max_seqlen_k.
 * Returns DSA_OK or DSA_ERR_BATCH (DSA_ERR_HIP if a copy fails). */
dsa_status dsa_check_batch(const dsa_batch* batch, hipStream_t stream);

/* Static description of a status code. */
const char* dsa_status_string(dsa_status status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int32_t dsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBDSA_DSA_H */

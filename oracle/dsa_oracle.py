"""Plain float64 / int64 NumPy oracle for the DSA hot path (test infrastructure only; see the
package docstring for who may call it).

Conventions (ragged batch):
  * ``cu_q`` [B+1]: queries of sequence b are rows cu_q[b] .. cu_q[b+1]-1.
  * ``cu_k`` [B+1]: key / latent rows of sequence b are rows cu_k[b] .. cu_k[b+1]-1, so its
    context length is L_b = cu_k[b+1] - cu_k[b].
  * query j of sequence b (nq_b = cu_q[b+1] - cu_q[b] new queries) sits at position
    p = L_b - nq_b + j and may look at sequence positions 0..p (itself included).
  * indices are sequence-local positions.
"""
from __future__ import annotations

import numpy as np


def query_positions(cu_q, cu_k):
    """For each query row t: (sequence b, position p, first key row of b)."""
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_k = np.asarray(cu_k, dtype=np.int64)
    out = []
    for b in range(len(cu_q) - 1):
        nq = int(cu_q[b + 1] - cu_q[b])
        L = int(cu_k[b + 1] - cu_k[b])
        if nq > L:
            raise ValueError(f"sequence {b}: {nq} queries but only {L} context rows")
        for j in range(nq):
            out.append((b, L - nq + j, int(cu_k[b])))
    return out


# ---------------------------------------------------------------------------------------------
# Step 1: lightning indexer.
# "How GLM5.3 Sparse Attention Affects HBM Memory Usage", How it works / Model: the score of a
# past token is a ReLU of a (down-projected) query-key dot product, summed with per-head
# weights across the indexer heads. The key is one row per token shared by all indexer heads;
# the heads live on the query side only.
#     I[t, s] = sum_j w[t, j] * max(0, q_I[t, j, :] . k_I[s, :])      for s = 0..p(t)
# No extra scale constant is applied: w carries any scaling.
# ---------------------------------------------------------------------------------------------
def indexer_scores_row(q_idx_t, k_rows, w_t):
    """Scores of one query against ``k_rows`` [n, d_I]: float64 [n]."""
    q = np.asarray(q_idx_t, dtype=np.float64)          # [H_I, d_I]
    k = np.asarray(k_rows, dtype=np.float64)           # [n, d_I]
    w = np.asarray(w_t, dtype=np.float64)              # [H_I]
    per_head = k @ q.T                                 # [n, H_I]: q_I[t,j] . k_I[s]
    return np.maximum(per_head, 0.0) @ w               # weighted sum of the ReLU over heads


def indexer_scores(q_idx, k_idx, w, cu_q, cu_k, rows=None):
    """Causal scores for the requested query rows (all rows by default).

    Returns {t: float64 array of length p(t)+1}.
    """
    pos = query_positions(cu_q, cu_k)
    rows = range(len(pos)) if rows is None else rows
    out = {}
    for t in rows:
        _, p, base = pos[t]
        out[t] = indexer_scores_row(q_idx[t], k_idx[base:base + p + 1], w[t])
    return out


# ---------------------------------------------------------------------------------------------
# Step 2: per-query causal top-k.
# "How GLM5.3 ...", How it works / Model: top-k is 2048 and below 2K tokens attention stays
# dense; the selection is shared across heads (one index row per query).
# Ties: scores compare as real numbers (so -0.0 equals +0.0) and an equal score goes to the
# lower position. The selected set is emitted in ascending position order, padded with -1.
# ---------------------------------------------------------------------------------------------
def topk_row(scores, k):
    """Top-``k`` positions of one causal score row (length n = p+1): int64 [k]."""
    s = np.asarray(scores, dtype=np.float64)
    n = s.shape[0]
    out = np.full(k, -1, dtype=np.int64)
    if n <= k:                                         # dense path: everything visible
        out[:n] = np.arange(n)
        return out
    # stable sort by descending score keeps ascending position among equal scores
    order = np.argsort(-s, kind="stable")
    out[:] = np.sort(order[:k])
    return out


def topk(score_rows, k):
    """{t: scores} -> {t: int64 [k] indices}."""
    return {t: topk_row(s, k) for t, s in score_rows.items()}


# ---------------------------------------------------------------------------------------------
# Step 2, block-pooled variant.
# "DeepSeek Sparse Attention" technique page, In the code: MiniMax-M3's lightning indexer pools
# its scores into blocks and keeps the top index_topk_blocks blocks per query; GLM-5.3-Flash's
# indexer scores pooled candidates. Reading taken: the visible scores of a query (positions
# 0..p) are cut into blocks of `block` consecutive positions (the last block holds the remainder);
# a block's score is the maximum, or the mean, of its visible scores; the k_blocks best blocks are
# chosen with the token-level rule (higher score first, an equal score going to the lower block,
# every block when at most k_blocks are visible); the query then attends to every visible position
# of the chosen blocks, emitted ascending and padded with -1 to k_blocks * block.
# A mean is a float64 quotient rounded once to fp32 before the blocks are compared: the selection
# is decided in the precision the kernel compares in (for integer-valued scores whose block sums
# stay below 2^24 the kernel's fp32 sum is exact and its fp32 quotient is that same rounding).
# ---------------------------------------------------------------------------------------------
def pool_blocks_row(scores, block, pool):
    """Block scores of one causal score row: float64 [ceil(n / block)]."""
    s = np.asarray(scores, dtype=np.float64)
    n = s.shape[0]
    nb = (n + block - 1) // block
    out = np.empty(nb)
    for c in range(nb):
        seg = s[c * block:min(n, (c + 1) * block)]
        if pool == "max":
            out[c] = seg.max()
        elif pool == "mean":
            out[c] = np.float64(np.float32(seg.sum() / seg.shape[0]))
        else:
            raise ValueError(pool)
    return out


def block_topk_row(scores, block, k_blocks, pool):
    """Positions attended by one query under block-pooled selection: int64 [k_blocks * block]."""
    n = np.asarray(scores).shape[0]
    chosen = topk_row(pool_blocks_row(scores, block, pool), k_blocks)
    out = np.full(k_blocks * block, -1, dtype=np.int64)
    pos = [np.arange(c * block, min(n, (c + 1) * block)) for c in chosen if c >= 0]
    if pos:
        pos = np.concatenate(pos)
        out[:pos.shape[0]] = pos
    return out


# ---------------------------------------------------------------------------------------------
# Step 3: sparse MLA in MQA mode.
# "How GLM5.3 ...", How it works / Model: all query heads attend, with softmax, over only the
# selected latent rows; the key of a row is its full latent+rope vector and (weight absorption)
# its value is the leading d_v columns of the same row.
#     z_s = scale * q[t,h,:] . kv[s,:]            s in S_t
#     o[t,h,:] = sum_s softmax(z)_s * kv[s,:d_v];  lse = logsumexp(z)
# ---------------------------------------------------------------------------------------------
def sparse_attention_row(q_t, kv_rows, d_v, scale):
    """One query (all heads) over the selected rows ``kv_rows`` [m, d_qk].

    Returns (o float64 [H, d_v], lse float64 [H]). With m = 0, o = 0 and lse = -inf.
    """
    q = np.asarray(q_t, dtype=np.float64)              # [H, d_qk]
    kv = np.asarray(kv_rows, dtype=np.float64)         # [m, d_qk]
    H = q.shape[0]
    if kv.shape[0] == 0:
        return np.zeros((H, d_v)), np.full(H, -np.inf)
    z = scale * (q @ kv.T)                             # [H, m]
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    l = e.sum(axis=1, keepdims=True)
    p = e / l
    o = p @ kv[:, :d_v]
    lse = (m + np.log(l))[:, 0]
    return o, lse


def sparse_attention(q, kv, indices, cu_q, cu_k, d_v, scale, rows=None):
    """Sparse MQA attention for the requested query rows; ``indices[t]`` holds sequence-local
    positions (-1 entries are skipped). Returns {t: (o, lse)}."""
    pos = query_positions(cu_q, cu_k)
    rows = range(len(pos)) if rows is None else rows
    out = {}
    for t in rows:
        _, _, base = pos[t]
        sel = np.asarray(indices[t], dtype=np.int64)
        sel = sel[sel >= 0]
        out[t] = sparse_attention_row(q[t], kv[base + sel], d_v, scale)
    return out


def dense_masked_attention_row(q_t, kv_seq, selected, d_v, scale):
    """The same attention written as dense softmax over the whole visible context with an
    additive mask: 0 on selected positions, -inf elsewhere ("DeepSeek Sparse Attention"
    technique page, In the code: selection applied as an additive sparse mask)."""
    q = np.asarray(q_t, dtype=np.float64)
    kv = np.asarray(kv_seq, dtype=np.float64)          # [n, d_qk] visible rows 0..p
    mask = np.full(kv.shape[0], -np.inf)
    sel = np.asarray(selected, dtype=np.int64)
    mask[sel[sel >= 0]] = 0.0
    z = scale * (q @ kv.T) + mask[None, :]
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    l = e.sum(axis=1, keepdims=True)
    return (e / l) @ kv[:, :d_v], (m + np.log(l))[:, 0]


# ---------------------------------------------------------------------------------------------
# Whole path and IndexShare.
# "How GLM5.3 ...", How it works / IndexShare: one indexer per group of DSA layers; its top-k
# indices are cached and reused by every layer of the group, each with its own queries and
# latent cache.
# ---------------------------------------------------------------------------------------------
def forward(q_idx, k_idx, w, q, kv, cu_q, cu_k, k, d_v, scale, rows=None):
    """Indexer -> top-k -> sparse attention for the requested rows.

    Returns (scores {t: array}, indices {t: int64 [k]}, attn {t: (o, lse)}).
    """
    scores = indexer_scores(q_idx, k_idx, w, cu_q, cu_k, rows)
    idx = topk(scores, k)
    attn = sparse_attention(q, kv, idx, cu_q, cu_k, d_v, scale, rows=list(idx.keys()))
    return scores, idx, attn


def index_share(q_idx, k_idx, w, q_layers, kv_layers, cu_q, cu_k, k, d_v, scale, rows=None):
    """One indexer + top-k pass whose indices feed every layer of the group.

    Returns (indices {t: [k]}, [ {t: (o, lse)} per layer ]).
    """
    scores = indexer_scores(q_idx, k_idx, w, cu_q, cu_k, rows)
    idx = topk(scores, k)
    outs = [sparse_attention(ql, kvl, idx, cu_q, cu_k, d_v, scale, rows=list(idx.keys()))
            for ql, kvl in zip(q_layers, kv_layers)]
    return idx, outs

"""CPU oracle for the DSA hot path — TEST INFRASTRUCTURE, NOT PRODUCT CODE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call anything in this package. The HIP library never uses it, and it shares no code
with the HIP path (no kernels, headers, helpers, tables or constants).

It is a plain, slow, obviously-correct NumPy implementation in float64 (int64 for indices) of
what the path computes, written from the pages' description of DeepSeek Sparse Attention:

* "How GLM5.3 Sparse Attention Affects HBM Memory Usage", section "How it works", part "Model":
  the lightning indexer scores tokens with a down-projected ReLU dot product summed with
  weights across heads; the selection is shared by all attention heads; sparse MLA runs in MQA
  mode over the top-k (k = 2048) tokens, and below 2K tokens attention stays dense.
* same page, part "IndexShare": every 4 DSA layers share one indexer and the cached top-k
  indices are reused by the shared layers.
* "DeepSeek Sparse Attention" technique page, table "In the code": the indexer is a weighted
  sum of ReLU(q.k) and queries attend only to the top index_topk tokens (the selection can be
  written as an additive sparse mask over dense attention); one variant pools the scores into
  blocks and keeps the top blocks (block_topk_row).

Every function states which of these it follows. Pins that tie the oracle to something other
than itself live in ``tests/test_oracle_pins.py``; the functions with no pin are listed there
as "parity unpinned" (none at present).
"""
from .dsa_oracle import (  # noqa: F401
    query_positions,
    indexer_scores_row,
    indexer_scores,
    topk_row,
    topk,
    pool_blocks_row,
    block_topk_row,
    sparse_attention_row,
    sparse_attention,
    dense_masked_attention_row,
    forward,
    index_share,
)

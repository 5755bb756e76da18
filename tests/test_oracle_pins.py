"""Pins that tie the CPU oracle to something other than itself (CPU only).

Each ``pin_*`` function checks the oracle against a fact fixed by the pages or by mathematics:
hand-worked examples (tests/golden, each with its derivation and citation), closed forms,
a library routine the method reduces to in a special case (dense causal attention via torch's
scaled_dot_product_attention when k covers the whole context), brute force on tiny inputs and
invariants. ``test_planted_mistakes_are_caught`` plants plausible mistakes in the oracle and
requires every one of them to fail at least one pin.

Parity unpinned: none.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle.dsa_oracle as O
from dsa_inputs import mixed_lengths

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f(x):
    return float(x)  # json strings like "-0.0" keep the sign of zero


# ------------------------------------------------------------------------------ indexer pins
def pin_indexer_worked():
    g = _load("indexer_worked.json")
    q = np.array(g["q_idx"], dtype=np.float64)
    k = np.array(g["k_idx"], dtype=np.float64)
    w = np.array(g["w"], dtype=np.float64)
    s = O.indexer_scores(q, k, w, g["cu_seqlens_q"], g["cu_seqlens_k"])
    for t, want in enumerate(g["scores"]):
        assert s[t].shape == (len(want),), (t, s[t].shape)
        assert np.array_equal(s[t], np.array(want, dtype=np.float64)), (t, s[t], want)
    for key, kk in (("top2", 2), ("top3", 3)):
        idx = O.topk(s, kk)
        for t, want in enumerate(g[key]):
            assert idx[t].tolist() == want, (key, t, idx[t], want)


def pin_indexer_one_hot_closed_form():
    # q_I[j] = a_j * e_{c_j} (a_j > 0) reduces the score to sum_j w_j * max(0, a_j * k[s, c_j])
    rng = np.random.default_rng(11)
    H, d, n = 5, 7, 19
    c = rng.integers(0, d, H)
    a = rng.integers(1, 4, H).astype(np.float64)
    q = np.zeros((H, d))
    q[np.arange(H), c] = a
    w = rng.integers(-3, 4, H).astype(np.float64)
    k = rng.integers(-5, 6, (n, d)).astype(np.float64)
    want = np.zeros(n)
    for s in range(n):
        for j in range(H):
            v = a[j] * k[s, c[j]]
            want[s] += w[j] * (v if v > 0 else 0.0)
    got = O.indexer_scores_row(q, k, w)
    assert np.array_equal(got, want), (got, want)


def pin_indexer_relu_identity():
    # relu(x) - relu(-x) = x, so I(q) - I(-q) = (sum_j w_j q_j) . k exactly (integer data)
    rng = np.random.default_rng(12)
    H, d, n = 6, 9, 23
    q = rng.integers(-4, 5, (H, d)).astype(np.float64)
    w = rng.integers(-2, 3, H).astype(np.float64)
    k = rng.integers(-4, 5, (n, d)).astype(np.float64)
    lhs = O.indexer_scores_row(q, k, w) - O.indexer_scores_row(-q, k, w)
    qsum = (w[:, None] * q).sum(axis=0)
    rhs = np.array([float(np.dot(qsum, k[s])) for s in range(n)])
    assert np.array_equal(lhs, rhs), (lhs, rhs)


def pin_indexer_invariants():
    rng = np.random.default_rng(13)
    H, d, n = 4, 8, 17
    q = rng.integers(-3, 4, (H, d)).astype(np.float64)
    k = rng.integers(-3, 4, (n, d)).astype(np.float64)
    w1 = rng.integers(-2, 3, H).astype(np.float64)
    w2 = rng.integers(-2, 3, H).astype(np.float64)
    f = O.indexer_scores_row
    assert np.array_equal(f(q, k, w1 + w2), f(q, k, w1) + f(q, k, w2))      # linear in w
    assert np.array_equal(f(2 * q, k, w1), 2 * f(q, k, w1))                  # homogeneous in q
    perm = rng.permutation(H)
    assert np.array_equal(f(q[perm], k, w1[perm]), f(q, k, w1))              # heads commute
    assert np.all(f(q, k, np.abs(w1)) >= 0)                                  # w >= 0 -> I >= 0
    # causal extent: query j of a sequence with nq queries over L rows sees p+1 = L-nq+j+1 rows
    cu_q, cu_k = [0, 3, 4], [0, 5, 12]
    qq = rng.integers(-3, 4, (4, H, d)).astype(np.float64)
    kk = rng.integers(-3, 4, (12, d)).astype(np.float64)
    ww = rng.integers(-2, 3, (4, H)).astype(np.float64)
    s = O.indexer_scores(qq, kk, ww, cu_q, cu_k)
    assert [len(s[t]) for t in range(4)] == [3, 4, 5, 7]
    # the last query of sequence 1 uses that sequence's own rows 5..11
    assert np.array_equal(s[3], f(qq[3], kk[5:12], ww[3]))


# -------------------------------------------------------------------------------- top-k pins
def pin_topk_worked():
    g = _load("topk_worked.json")
    for case in g["cases"]:
        got = O.topk_row(np.array([_f(x) for x in case["scores"]]), case["k"])
        assert got.tolist() == case["expect"], (case, got)


def _topk_by_rank(s, k):
    """Definition by counting: s_i is selected iff fewer than k positions beat it, where u
    beats i when s_u > s_i, or s_u == s_i and u < i."""
    n = len(s)
    if n <= k:
        return list(range(n)) + [-1] * (k - n)
    sel = [i for i in range(n)
           if sum(1 for u in range(n) if s[u] > s[i] or (s[u] == s[i] and u < i)) < k]
    return sel


def pin_topk_brute_force():
    rng = np.random.default_rng(21)
    for trial in range(300):
        n = int(rng.integers(1, 40))
        k = int(rng.integers(1, 12))
        span = int(rng.integers(1, 6))            # small spans force heavy ties
        s = rng.integers(-span, span + 1, n).astype(np.float64)
        s[rng.random(n) < 0.2] *= -1.0           # flips some zeros to -0.0
        got = O.topk_row(s, k).tolist()
        assert got == _topk_by_rank(s, k), (trial, s, k, got)


def pin_topk_special_cases():
    k = 16
    n = 100
    assert O.topk_row(np.full(n, 3.0), k).tolist() == list(range(k))          # all equal
    assert O.topk_row(np.arange(n, dtype=float), k).tolist() == list(range(n - k, n))
    assert O.topk_row(np.arange(5, dtype=float), k).tolist() == list(range(5)) + [-1] * (k - 5)
    rng = np.random.default_rng(22)
    s = rng.normal(size=n)
    idx = O.topk_row(s, k)
    assert np.all(np.diff(idx) > 0) and idx.min() >= 0 and idx.max() < n
    unsel = np.setdiff1d(np.arange(n), idx)
    assert s[idx].min() >= s[unsel].max()


# ---------------------------------------------------------------------------- attention pins
def pin_attention_worked():
    g = _load("attention_worked.json")
    kv = np.array(g["kv"], dtype=np.float64)
    sel = np.array(g["selected"])
    for case in g["cases"]:
        o, lse = O.sparse_attention_row(np.array(case["q"]), kv[sel], g["d_v"], case["scale"])
        assert np.allclose(o, np.array(case["o"]), rtol=0, atol=1e-12), (o, case["o"])
        assert np.allclose(lse, np.array(case["lse"]), rtol=0, atol=1e-12), (lse, case["lse"])
        # the same through the batched entry (one sequence, query at the last position)
        idx = np.full((1, 5), -1)
        idx[0, :3] = sel
        out = O.sparse_attention(np.array(case["q"])[None], kv, idx, [0, 1], [0, 4], g["d_v"],
                                 case["scale"])
        assert np.allclose(out[0][0], np.array(case["o"]), rtol=0, atol=1e-12)


def _sdpa_reference(q, kv, cu_q, cu_k, d_v, scale):
    """Dense causal MQA attention through torch's scaled_dot_product_attention (float64, CPU):
    one shared key/value for every head, query j of a sequence at position L-nq+j."""
    outs = []
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        nq, L = q1 - q0, k1 - k0
        qb = torch.from_numpy(q[q0:q1]).permute(1, 0, 2)[None]           # [1,H,nq,d_qk]
        H = qb.shape[1]
        kb = torch.from_numpy(kv[k0:k1]).contiguous()
        K = kb[None, None].expand(1, H, L, kb.shape[1])
        V = kb[:, :d_v].contiguous()[None, None].expand(1, H, L, d_v)
        pos = torch.arange(nq)[:, None] + (L - nq)
        mask = torch.arange(L)[None, :] <= pos                            # bottom-right causal
        o = torch.nn.functional.scaled_dot_product_attention(qb, K, V, attn_mask=mask,
                                                             scale=scale)
        outs.append(o[0].permute(1, 0, 2).numpy())
    return np.concatenate(outs, axis=0)


def pin_attention_dense_equals_sdpa():
    rng = np.random.default_rng(31)
    for cu_q, cu_k in (([0, 12], [0, 12]),              # prefill: every row attends to itself
                       ([0, 1, 3, 6], [0, 9, 20, 26])):  # decode / chunked rows, ragged
        T, L = cu_q[-1], cu_k[-1]
        H, d_qk, d_v = 3, 10, 6
        q = rng.normal(size=(T, H, d_qk))
        kv = rng.normal(size=(L, d_qk))
        q_idx = rng.integers(-3, 4, (T, 2, 4)).astype(np.float64)
        k_idx = rng.integers(-3, 4, (L, 4)).astype(np.float64)
        w = rng.integers(-2, 3, (T, 2)).astype(np.float64)
        scale = 1.0 / math.sqrt(d_qk)
        kmax = max(cu_k[b + 1] - cu_k[b] for b in range(len(cu_k) - 1))
        _, idx, attn = O.forward(q_idx, k_idx, w, q, kv, cu_q, cu_k, kmax, d_v, scale)
        ref = _sdpa_reference(q, kv, cu_q, cu_k, d_v, scale)
        got = np.stack([attn[t][0] for t in range(T)])
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-12), np.abs(got - ref).max()


def pin_attention_mask_form():
    rng = np.random.default_rng(32)
    H, d_qk, d_v, n = 4, 12, 8, 30
    for _ in range(10):
        q = rng.normal(size=(H, d_qk))
        kv = rng.normal(size=(n, d_qk))
        m = int(rng.integers(1, n + 1))
        sel = np.sort(rng.choice(n, m, replace=False))
        o1, l1 = O.sparse_attention_row(q, kv[sel], d_v, 0.3)
        o2, l2 = O.dense_masked_attention_row(q, kv, sel, d_v, 0.3)
        assert np.allclose(o1, o2, rtol=1e-12, atol=1e-12)
        assert np.allclose(l1, l2, rtol=1e-12, atol=1e-12)


def pin_attention_invariants():
    rng = np.random.default_rng(33)
    H, d_qk, d_v, m = 5, 16, 12, 40
    q = rng.normal(size=(H, d_qk))
    kv = rng.normal(size=(m, d_qk))
    o, lse = O.sparse_attention_row(q, kv, d_v, 0.25)
    perm = rng.permutation(m)
    o2, lse2 = O.sparse_attention_row(q, kv[perm], d_v, 0.25)        # order of the set
    assert np.allclose(o, o2, rtol=1e-12, atol=1e-12) and np.allclose(lse, lse2, rtol=1e-12)
    o1, _ = O.sparse_attention_row(q, kv[3:4], d_v, 0.25)             # one visible row
    assert np.array_equal(o1, np.repeat(kv[3:4, :d_v], H, axis=0))
    kv1 = kv.copy()
    kv1[:, :d_v] = 1.0                                                # V == 1 -> output 1
    o3, _ = O.sparse_attention_row(q, kv1, d_v, 0.25)
    assert np.allclose(o3, 1.0, rtol=0, atol=1e-13)
    # lse is logsumexp of the scaled logits
    z = 0.25 * (q @ kv.T)
    assert np.allclose(lse, np.log(np.exp(z).sum(axis=1)), rtol=1e-12)


# ------------------------------------------------------------------ block-pooled selection pins
def pin_block_topk_worked():
    g = _load("block_topk_worked.json")
    for c in g["cases"]:
        s = np.array([_f(x) for x in c["scores"]])
        for pool in ("max", "mean"):
            got = O.block_topk_row(s, c["block"], c["k"], pool)
            assert got.tolist() == c[pool], (c["why"], pool, got.tolist())


def pin_block_topk_block1_is_token_topk():
    # blocks of one position: every pooling is the score itself, so the selection is top-k
    rng = np.random.default_rng(31)
    for _ in range(60):
        n = int(rng.integers(1, 200))
        s = rng.integers(-4, 5, n).astype(np.float64)
        k = int(rng.integers(1, 40))
        want = O.topk_row(s, k)
        for pool in ("max", "mean"):
            assert np.array_equal(O.block_topk_row(s, 1, k, pool), want), (n, k, pool)


def pin_block_topk_brute_force():
    # block c is chosen iff fewer than k blocks beat it (a higher pooled score, or an equal one
    # at a lower block), or every block is chosen when at most k are visible; the output is the
    # chosen blocks' visible positions, ascending
    rng = np.random.default_rng(37)
    for _ in range(200):
        n = int(rng.integers(1, 300))
        block = int(rng.choice([2, 3, 4, 8, 16]))
        k = int(rng.integers(1, 12))
        s = rng.integers(-3, 4, n).astype(np.float64)
        for pool in ("max", "mean"):
            J = O.pool_blocks_row(s, block, pool)
            nb = J.shape[0]
            chosen = [c for c in range(nb)
                      if nb <= k or sum(1 for d in range(nb)
                                        if J[d] > J[c] or (J[d] == J[c] and d < c)) < k]
            want = [x for c in chosen for x in range(c * block, min(n, (c + 1) * block))]
            got = O.block_topk_row(s, block, k, pool)
            assert got[:len(want)].tolist() == want and (got[len(want):] == -1).all(), \
                (n, block, k, pool)
            assert got.shape == (k * block,)


def pin_block_topk_invariants():
    rng = np.random.default_rng(41)
    for _ in range(100):
        n = int(rng.integers(2, 400))
        block = int(rng.choice([4, 8, 16, 64]))
        k = int(rng.integers(1, 8))
        s = rng.integers(-6, 7, n).astype(np.float64)
        for pool in ("max", "mean"):
            base = O.block_topk_row(s, block, k, pool)
            # the pooled score of a block does not depend on the order inside it
            p = s.copy()
            for c in range(0, n, block):
                seg = p[c:c + block]
                p[c:c + block] = seg[rng.permutation(seg.shape[0])]
            assert np.array_equal(O.block_topk_row(p, block, k, pool), base)
            # nor on a constant added to every score
            assert np.array_equal(O.block_topk_row(s + 5.0, block, k, pool), base)
        # max pooling always keeps the block of the best-scoring position
        top = int(np.argmax(s)) // block
        chosen = set(x // block for x in O.block_topk_row(s, block, k, "max") if x >= 0)
        assert top in chosen


# --------------------------------------------------------------------------- IndexShare pin
def pin_index_share():
    rng = np.random.default_rng(41)
    cu_q, cu_k = [0, 1, 2], [0, 50, 90]
    T, L = 2, 90
    q_idx = rng.integers(-3, 4, (T, 2, 4)).astype(np.float64)
    k_idx = rng.integers(-3, 4, (L, 4)).astype(np.float64)
    w = rng.integers(-2, 3, (T, 2)).astype(np.float64)
    qs = [rng.normal(size=(T, 3, 6)) for _ in range(4)]
    kvs = [rng.normal(size=(L, 6)) for _ in range(4)]
    # count the (query, key) score pairs the indexer evaluates
    import oracle.dsa_oracle as mod
    pairs = [0]
    real_row = mod.indexer_scores_row

    def counting_row(q, k, w_):
        pairs[0] += len(k)
        return real_row(q, k, w_)

    mod.indexer_scores_row = counting_row
    try:
        idx, outs = O.index_share(q_idx, k_idx, w, qs, kvs, cu_q, cu_k, 8, 4, 0.4)
        shared_pairs = pairs[0]
        pairs[0] = 0
        per_layer = []
        for layer in range(4):
            per_layer.append(O.forward(q_idx, k_idx, w, qs[layer], kvs[layer], cu_q, cu_k, 8, 4,
                                       0.4))
        separate_pairs = pairs[0]
    finally:
        mod.indexer_scores_row = real_row
    for layer, (_, idx_l, attn_l) in enumerate(per_layer):
        for t in range(T):
            assert np.array_equal(idx[t], idx_l[t])          # one selection for the group
            assert np.array_equal(outs[layer][t][0], attn_l[t][0])
    # causal pairs of the two queries (positions 49 and 39): 50 + 40. The group evaluates them
    # once; one indexer per layer would evaluate them four times, so sharing cuts the indexer
    # work by 75%
    assert shared_pairs == 90
    assert separate_pairs == 4 * 90
    assert 1 - shared_pairs / separate_pairs == 0.75


ALL_PINS = [pin_indexer_worked, pin_indexer_one_hot_closed_form, pin_indexer_relu_identity,
            pin_indexer_invariants, pin_topk_worked, pin_topk_brute_force,
            pin_topk_special_cases, pin_attention_worked, pin_attention_dense_equals_sdpa,
            pin_attention_mask_form, pin_attention_invariants, pin_index_share,
            pin_block_topk_worked, pin_block_topk_block1_is_token_topk,
            pin_block_topk_brute_force, pin_block_topk_invariants]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


# ------------------------------------------------------------------ planted mistakes (CPU)
def _m_no_relu(q, k, w):
    return (np.asarray(k, float) @ np.asarray(q, float).T) @ np.asarray(w, float)


def _m_relu_after_weight(q, k, w):
    x = np.asarray(k, float) @ np.asarray(q, float).T
    return np.maximum(x * np.asarray(w, float)[None, :], 0).sum(axis=1)


def _m_unweighted(q, k, w):
    x = np.asarray(k, float) @ np.asarray(q, float).T
    return np.maximum(x, 0).sum(axis=1)


def _m_topk_ties_high(s, k):
    s = np.asarray(s, float)
    n = len(s)
    if n <= k:
        return np.concatenate([np.arange(n), -np.ones(k - n, int)])
    order = np.lexsort((-np.arange(n), -s))          # equal scores: higher position first
    return np.sort(order[:k])


def _m_topk_unsorted(s, k):
    s = np.asarray(s, float)
    n = len(s)
    if n <= k:
        return np.concatenate([np.arange(n), -np.ones(k - n, int)])
    return np.argsort(-s, kind="stable")[:k]         # forgets the ascending emission


def _m_topk_dense_pad_zero(s, k):
    s = np.asarray(s, float)
    n = len(s)
    if n <= k:
        return np.concatenate([np.arange(n), np.zeros(k - n, int)])   # pads with 0, not -1
    return np.sort(np.argsort(-s, kind="stable")[:k])


def _attn_variant(drop_rope=False, v_offset=0, no_scale=False, lse_without_max=False):
    def f(q, kv_rows, d_v, scale):
        q = np.asarray(q, float)
        kv = np.asarray(kv_rows, float)
        kq = kv.copy()
        if drop_rope:
            kq[:, d_v:] = 0.0
        z = (1.0 if no_scale else scale) * (q @ kq.T)
        m = z.max(axis=1, keepdims=True)
        e = np.exp(z - m)
        l = e.sum(axis=1, keepdims=True)
        v = kv[:, v_offset:v_offset + d_v]
        if v.shape[1] < d_v:
            v = np.pad(v, ((0, 0), (0, d_v - v.shape[1])))
        lse = np.log(l)[:, 0] if lse_without_max else (m + np.log(l))[:, 0]
        return (e / l) @ v, lse
    return f


def _m_positions_exclusive(cu_q, cu_k):
    out = []
    for b in range(len(cu_q) - 1):
        nq = int(cu_q[b + 1] - cu_q[b])
        L = int(cu_k[b + 1] - cu_k[b])
        for j in range(nq):
            out.append((b, L - nq + j - 1, int(cu_k[b])))   # forgets that a query sees itself
    return out


def _m_positions_wrong_base(cu_q, cu_k):
    out = []
    for b in range(len(cu_q) - 1):
        nq = int(cu_q[b + 1] - cu_q[b])
        L = int(cu_k[b + 1] - cu_k[b])
        for j in range(nq):
            out.append((b, L - nq + j, 0))                   # every sequence reads rows from 0
    return out


def _m_pool_shifted_boundaries(scores, block, pool):
    s = np.asarray(scores, float)
    n = s.shape[0]
    nb = (n + block - 1) // block
    out = np.empty(nb)
    for c in range(nb):                                # blocks start one position late
        seg = s[min(n - 1, c * block + 1):min(n, (c + 1) * block + 1)]
        out[c] = seg.max() if pool == "max" else seg.mean()
    return out


def _m_pool_mean_over_whole_block(scores, block, pool):
    s = np.asarray(scores, float)
    n = s.shape[0]
    nb = (n + block - 1) // block
    out = np.empty(nb)
    for c in range(nb):                                # the last block divides by `block`
        seg = s[c * block:min(n, (c + 1) * block)]
        out[c] = seg.max() if pool == "max" else seg.sum() / block
    return out


def _m_pool_ignores_kind(scores, block, pool):
    s = np.asarray(scores, float)
    n = s.shape[0]
    return np.array([s[c:min(n, c + block)].mean() for c in range(0, n, block)])


def _m_block_drops_partial_block(scores, block, k_blocks, pool):
    n = np.asarray(scores).shape[0]
    chosen = O.topk_row(O.pool_blocks_row(scores, block, pool), k_blocks)
    out = np.full(k_blocks * block, -1, dtype=np.int64)
    pos = [np.arange(c * block, (c + 1) * block) for c in chosen
           if c >= 0 and (c + 1) * block <= n]         # forgets the remainder block
    if pos:
        pos = np.concatenate(pos)
        out[:pos.shape[0]] = pos
    return out


MUTANTS = {
    "indexer_no_relu": ("indexer_scores_row", _m_no_relu),
    "indexer_relu_after_weight": ("indexer_scores_row", _m_relu_after_weight),
    "indexer_unweighted": ("indexer_scores_row", _m_unweighted),
    "topk_ties_to_higher_index": ("topk_row", _m_topk_ties_high),
    "topk_not_ascending": ("topk_row", _m_topk_unsorted),
    "topk_dense_pads_with_zero": ("topk_row", _m_topk_dense_pad_zero),
    "attention_drops_rope_columns": ("sparse_attention_row", _attn_variant(drop_rope=True)),
    "attention_value_from_wrong_slice": ("sparse_attention_row", _attn_variant(v_offset=1)),
    "attention_ignores_scale": ("sparse_attention_row", _attn_variant(no_scale=True)),
    "attention_lse_without_max": ("sparse_attention_row", _attn_variant(lse_without_max=True)),
    "causal_excludes_self": ("query_positions", _m_positions_exclusive),
    "ragged_base_ignored": ("query_positions", _m_positions_wrong_base),
    "block_boundaries_shifted": ("pool_blocks_row", _m_pool_shifted_boundaries),
    "block_mean_divides_by_block": ("pool_blocks_row", _m_pool_mean_over_whole_block),
    "block_pool_always_mean": ("pool_blocks_row", _m_pool_ignores_kind),
    "block_remainder_dropped": ("block_topk_row", _m_block_drops_partial_block),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_are_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    caught = []
    for pin in ALL_PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"planted mistake {name} passed every pin"


# ------------------------------------------------------------------------ workload recipe
def test_mixed_lengths_recipe():
    lens = mixed_lengths()
    assert lens == [14109, 74042, 237082, 772, 1042009, 3060, 4525, 9522, 742, 26042, 861235,
                    512, 11530, 723, 1048576, 242453]
    assert sum(lens) == 3576934
    assert sorted(x for x in lens if x <= 2048) == [512, 723, 742, 772]   # dense-path rows


def test_byte_model_closed_forms():
    # decode intensity of MQA sparse MLA over a bf16 576-wide latent row, 64 heads, the value
    # being its leading 512 columns: 64 * 2 * (576 + 512) FLOP per 1152 B row
    assert abs(64 * 2 * (576 + 512) / (576 * 2) - 120.8) < 0.1
    # a separate 512-wide value row (1088 stored columns) would give 64 FLOP/B instead
    assert 64 * 2 * (576 + 512) / ((576 + 512) * 2) == 64.0
    # latent cache of the 1M-token sequence: ~1.2 GB per layer
    assert abs(1048576 * 576 * 2 / 1e9 - 1.2) < 0.01

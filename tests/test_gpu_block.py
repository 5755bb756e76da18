"""GPU parity of the block-pooled selection (dsa_block_topk) against the CPU oracle.

Indices are compared bit for bit with the oracle's block_topk_row on the same score rows. Max
pooling is exact for any scores; mean pooling is compared on integer-valued scores (every
workload's scores are integers), whose fp32 block sums are exact. The attention over the chosen
positions is compared with the oracle per query.
"""
import sys
import zlib

import numpy as np
import pytest
import torch

import dsa_inputs as DI
import long_context_lightning_amd as dsa
import oracle.dsa_oracle as O
from tolerance import attn_close

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsa.lib()


def host64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def batch_of(case, d):
    return dsa.Batch(d["cu_seqlens_q"], d["cu_seqlens_k"], max(case.seqlens_q),
                     max(case.seqlens_k), case.total_q, case.total_k)


def check_rows(case, scores, idx, block, kb, pool, rows=None):
    qrows = DI.query_rows(case)
    rows = range(case.total_q) if rows is None else rows
    for t in rows:
        p = qrows[t][2]
        want = O.block_topk_row(scores[t, :p + 1].double().cpu().numpy(), block, kb, pool)
        got = idx[t].cpu().numpy().astype(np.int64)
        assert np.array_equal(got, want), (t, pool, block, kb, np.sum(got != want))


@pytest.mark.parametrize("name", ["decode_b32_l16k", "indexshare_b8_l256k", "mixed_b16_l512_1m"])
@pytest.mark.parametrize("pool", ["max", "mean"])
def test_block_topk_workloads_all_rows(name, pool):
    case = DI.CASES[name]
    say("case", case.name, pool)
    d = DI.make_inputs(case, "cuda", layers=1)
    batch = batch_of(case, d)
    scores = dsa.indexer_scores(d["q_idx"], d["k_idx"], d["w"], batch)
    idx = dsa.block_topk(scores, batch, 64, 32, pool)
    torch.cuda.synchronize()
    check_rows(case, scores, idx, 64, 32, pool)


def test_block_topk_chunked_prefill_sampled_rows():
    case = DI.CASES["prefill_chunk8k_l64k"]
    d = DI.make_inputs(case, "cuda", layers=1)
    batch = batch_of(case, d)
    scores = dsa.indexer_scores(d["q_idx"], d["k_idx"], d["w"], batch)
    for pool in ("max", "mean"):
        idx = dsa.block_topk(scores, batch, 64, 32, pool)
        torch.cuda.synchronize()
        T = case.total_q
        check_rows(case, scores, idx, 64, 32, pool,
                   sorted(set([0, 1, 63, 64, 65, T - 1] + list(range(7, T, 61)))))


@pytest.mark.parametrize("block,kb", [(4, 100), (8, 3), (16, 128), (32, 64), (128, 16), (256, 8),
                                      (64, 1), (64, 1024)])
def test_block_topk_sizes_and_edges(block, kb):
    name = f"blk_{block}_{kb}"
    lens = (1, 5, block, block + 1, kb * block, kb * block + 1, 3 * kb * block + 7, 20000)
    case = DI.custom_case(name, lens, (1, 1, 1, 1, 1, 1, 2, 3),
                          seed_base=zlib.crc32(name.encode()) % 100000 * 100)
    d = DI.make_inputs(case, "cuda", layers=1)
    batch = batch_of(case, d)
    scores = dsa.indexer_scores(d["q_idx"], d["k_idx"], d["w"], batch)
    for pool in ("max", "mean"):
        idx = dsa.block_topk(scores, batch, block, kb, pool)
        torch.cuda.synchronize()
        check_rows(case, scores, idx, block, kb, pool)


def test_block_topk_crafted_rows():
    """Explicit score rows: heavy ties, every block equal, one outlier, signed zeros, floats
    (max pooling, exact for any scores) and integers (both poolings)."""
    rng = np.random.default_rng(8)
    rows_int = [rng.integers(-1, 2, 30000), np.zeros(9000), np.arange(5000) % 7,
                np.repeat(rng.integers(-3, 4, 300), 64)[:19000]]
    rows_flt = [rng.normal(size=40000), np.where(rng.random(12000) < 0.5, 0.0, -0.0),
                np.concatenate([rng.normal(size=7000), [1e30], rng.normal(size=9000)])]
    for rows, pools in ((rows_int, ("max", "mean")), (rows_flt, ("max",))):
        lens = [len(r) for r in rows]
        batch = dsa.Batch.from_lengths([1] * len(lens), lens)
        sc = torch.zeros((len(lens), max(lens)), dtype=torch.float32)
        for i, r in enumerate(rows):
            sc[i, :len(r)] = torch.from_numpy(np.asarray(r, dtype=np.float32))
        sc = sc.cuda()
        for pool in pools:
            for block, kb in ((64, 32), (16, 50)):
                idx = dsa.block_topk(sc, batch, block, kb, pool)
                torch.cuda.synchronize()
                for i, r in enumerate(rows):
                    want = O.block_topk_row(np.asarray(r, dtype=np.float32).astype(np.float64),
                                            block, kb, pool)
                    got = idx[i].cpu().numpy().astype(np.int64)
                    assert np.array_equal(got, want), (i, pool, block, kb)


def test_block_selection_feeds_sparse_mla():
    """indexer -> block selection -> sparse MLA over the chosen runs of rows; each query's output
    against the oracle's attention over the oracle's block selection."""
    case = DI.custom_case("blk_attn", (16384, 5000, 30000, 1500), (1, 1, 2, 1),
                          seed_base=zlib.crc32(b"blk_attn") % 100000 * 100)
    d = DI.make_inputs(case, "cuda")
    batch = batch_of(case, d)
    scores = dsa.indexer_scores(d["q_idx"], d["k_idx"], d["w"], batch)
    idx = dsa.block_topk(scores, batch, 64, 32, "max")
    out, lse = dsa.sparse_mla_fwd(d["q"][0], d["kv"][0], idx, batch, case.softmax_scale, case.d_v)
    torch.cuda.synchronize()
    for t, b, p, base in DI.query_rows(case):
        s = O.indexer_scores_row(host64(d["q_idx"][t]), host64(d["k_idx"][base:base + p + 1]),
                                 host64(d["w"][t]))
        sel = O.block_topk_row(s, 64, 32, "max")
        assert np.array_equal(idx[t].cpu().numpy().astype(np.int64), sel), t
        rows = torch.as_tensor(sel[sel >= 0], device="cuda") + base
        o, l = O.sparse_attention_row(host64(d["q"][0][t]), host64(d["kv"][0][rows]), case.d_v,
                                      case.softmax_scale)
        ok, a, r = attn_close(out[t].float().cpu().numpy(), o)
        assert ok, (t, a, r)


def test_forward_with_block_selection():
    """dsa_forward with block_size > 0: the shared indices are dsa_block_topk's, the outputs
    those of the separate calls, bit for bit, and a reusing layer reads the same indices."""
    case = DI.custom_case("blk_fwd", (16384, 9000, 2000, 40000), (1, 1, 1, 1), layers=2,
                          seed_base=zlib.crc32(b"blk_fwd") % 100000 * 100)
    d = DI.make_inputs(case, "cuda")
    batch = batch_of(case, d)
    for pool in ("max", "mean"):
        shared = None
        outs = []
        for l in range(case.layers):
            o, _, shared = dsa.forward(d["q"][l], d["kv"][l], batch, case.index_topk,
                                       case.softmax_scale, case.d_v, q_idx=d["q_idx"],
                                       k_idx=d["k_idx"], w=d["w"], shared_indices=shared,
                                       compute_indices=(l == 0), block_size=64, pool=pool)
            outs.append(o)
        scores = dsa.indexer_scores(d["q_idx"], d["k_idx"], d["w"], batch)
        idx = dsa.block_topk(scores, batch, 64, case.index_topk // 64, pool)
        torch.cuda.synchronize()
        assert torch.equal(idx, shared), pool
        check_rows(case, scores, idx, 64, case.index_topk // 64, pool)
        for l in range(case.layers):
            o, _ = dsa.sparse_mla_fwd(d["q"][l], d["kv"][l], idx, batch, case.softmax_scale,
                                      case.d_v)
            torch.cuda.synchronize()
            assert torch.equal(o, outs[l]), (pool, l)

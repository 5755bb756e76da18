"""GPU parity of the fp8 (OCP e4m3fn) lightning indexer against the CPU oracle.

The indexer inputs of every workload are integers in [-4, 4], which e4m3fn holds exactly, so the
fp8 path must give the same scores as the oracle bit for bit (products are exact and every
partial sum is an integer below 2^24), and the same top-k indices. Key scales are powers of two
here, so the scaled scores stay exact; the oracle receives the dequantised keys k * scale.
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


def fp8(t):
    out = t.to(torch.float8_e4m3fn)
    assert torch.equal(out.float(), t.float()), "inputs must be exact in e4m3fn"
    return out


def pow2_scales(n, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    e = torch.randint(-2, 3, (n,), generator=g, device="cuda").float()
    return torch.exp2(e)


def check_scores_and_topk(case, d, scores, idx, k_scale=None, rows=None):
    """Every requested row: scores bit-exact against the oracle on the dequantised keys, and
    indices equal to the oracle's top-k."""
    qrows = DI.query_rows(case)
    rows = range(case.total_q) if rows is None else rows
    for t in rows:
        _, b, p, base = qrows[t]
        k_rows = host64(d["k_idx"][base:base + p + 1])
        if k_scale is not None:
            k_rows = k_rows * host64(k_scale[base:base + p + 1])[:, None]
        ref = O.indexer_scores_row(host64(d["q_idx"][t]), k_rows, host64(d["w"][t]))
        got = scores[t, :p + 1].double().cpu().numpy()
        bad = np.nonzero(got != ref)[0]
        assert bad.size == 0, f"row {t}: {bad.size} score mismatches, first at {bad[:5]}"
        want = O.topk_row(ref, case.index_topk)
        assert np.array_equal(idx[t].cpu().numpy().astype(np.int64), want), f"row {t} indices"


@pytest.mark.parametrize("name", ["decode_b32_l16k", "indexshare_b8_l256k", "mixed_b16_l512_1m",
                                  "mtp_b32_l16k_q4_shared"])
def test_fp8_indexer_workloads_all_rows(name):
    case = DI.CASES[name]
    say("case", case.name)
    d = DI.make_inputs(case, "cuda", layers=1)
    batch = batch_of(case, d)
    qf, kf = fp8(d["q_idx"]), fp8(d["k_idx"])
    scores = dsa.indexer_scores_fp8(qf, kf, d["w"], batch)
    idx = dsa.topk(scores, batch, case.index_topk)
    ref_scores = dsa.indexer_scores(d["q_idx"], d["k_idx"], d["w"], batch)
    torch.cuda.synchronize()
    # the bf16 and fp8 paths are both exact: identical on every valid entry
    for t, b, p, base in DI.query_rows(case):
        assert torch.equal(scores[t, :p + 1], ref_scores[t, :p + 1]), f"row {t}"
    check_scores_and_topk(case, d, scores, idx)


def test_fp8_indexer_key_scales():
    case = DI.custom_case("fp8_scaled", (16384, 3000, 40000, 700, 9000), (1, 2, 1, 3, 1),
                          seed_base=zlib.crc32(b"fp8_scaled") % 100000 * 100)
    d = DI.make_inputs(case, "cuda", layers=1)
    batch = batch_of(case, d)
    ks = pow2_scales(case.total_k, 17)
    scores = dsa.indexer_scores_fp8(fp8(d["q_idx"]), fp8(d["k_idx"]), d["w"], batch, k_scale=ks)
    idx = dsa.topk(scores, batch, case.index_topk)
    torch.cuda.synchronize()
    check_scores_and_topk(case, d, scores, idx, k_scale=ks)


@pytest.mark.parametrize("lens,nq,heads", [
    ((1,), (1,), 32),
    ((2047, 2048, 2049, 2050), (1, 1, 1, 1), 32),
    ((37, 3000, 5, 9000, 65), (1, 2, 1, 3, 4), 32),
    ((300, 129), (40, 17), 32),            # many queries per sequence
    ((5000, 700, 12000), (1, 1, 2), 64),   # 64 indexer heads
    ((9000, 7, 3000, 20000), (7, 7, 5, 15), 32),   # token groups of four, partial last groups
])
def test_fp8_indexer_edge_cases(lens, nq, heads):
    name = f"fp8_edge_{lens}_{nq}_{heads}"
    case = DI.custom_case(name, lens, nq, index_n_heads=heads,
                          seed_base=zlib.crc32(name.encode()) % 100000 * 100)
    d = DI.make_inputs(case, "cuda", layers=1)
    batch = batch_of(case, d)
    scores = dsa.indexer_scores_fp8(fp8(d["q_idx"]), fp8(d["k_idx"]), d["w"], batch)
    idx = dsa.topk(scores, batch, case.index_topk)
    torch.cuda.synchronize()
    check_scores_and_topk(case, d, scores, idx)


def test_fp8_forward_indexshare_matches_bf16_path():
    """The fused call with the fp8 indexer: cached indices equal the bf16 path's, and every layer's
    output is bit-identical to the bf16-indexer forward (the attention is the same bf16 kernel
    over the same indices); outputs against the oracle per query."""
    case = DI.custom_case("fp8_fwd", (9000, 20000, 4000, 16384), (1, 1, 1, 1), layers=2,
                          seed_base=zlib.crc32(b"fp8_fwd") % 100000 * 100)
    d = DI.make_inputs(case, "cuda")
    batch = batch_of(case, d)
    qf, kf = fp8(d["q_idx"]), fp8(d["k_idx"])
    ks = pow2_scales(case.total_k, 5)
    shared = None
    outs = []
    for l in range(case.layers):
        o, ls, shared = dsa.forward(d["q"][l], d["kv"][l], batch, case.index_topk,
                                    case.softmax_scale, case.d_v, q_idx=qf, k_idx=kf, w=d["w"],
                                    k_idx_scale=ks, shared_indices=shared,
                                    compute_indices=(l == 0))
        outs.append(o)
    scores = dsa.indexer_scores_fp8(qf, kf, d["w"], batch, k_scale=ks)
    idx = dsa.topk(scores, batch, case.index_topk)
    torch.cuda.synchronize()
    assert torch.equal(idx, shared)
    check_scores_and_topk(case, d, scores, idx, k_scale=ks)
    for l in range(case.layers):
        o, _ = dsa.sparse_mla_fwd(d["q"][l], d["kv"][l], idx, batch, case.softmax_scale, case.d_v)
        torch.cuda.synchronize()
        assert torch.equal(o, outs[l])
        for t, b, p, base in DI.query_rows(case):
            sel = idx[t][idx[t] >= 0].long()
            ref, _ = O.sparse_attention_row(host64(d["q"][l][t]), host64(d["kv"][l][base + sel]),
                                            case.d_v, case.softmax_scale)
            ok, a, r = attn_close(outs[l][t].float().cpu().numpy(), ref)
            assert ok, (l, t, a, r)

"""GPU parity: libdsa (through the C ABI) against the CPU oracle on the same seeded inputs.

Bar: indexer scores and top-k indices bit-exact (integer-valued indexer inputs make every fp32
score exact); attention outputs within max|d| <= 2e-2 and ||d||/||ref|| <= 1e-2 (tolerance.py),
applied to every query (and layer) on its own. Every workload is compared on every row, except
that the chunked prefill (8192 rows over 64K keys) compares scores and outputs on 264 rows
spread over the chunk and the indices of every row with the oracle's top-k of the row's scores.
"""
import math
import sys
import zlib

import numpy as np
import pytest
import torch

import dsa_inputs as DI
import long_context_lightning_amd as dsa
import oracle.dsa_oracle as O
from tolerance import attn_close, attn_errors

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsa.lib()  # fail loudly if libdsa.so is missing


def host64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def batch_of(case, d):
    return dsa.Batch(d["cu_seqlens_q"], d["cu_seqlens_k"], max(case.seqlens_q),
                     max(case.seqlens_k), case.total_q, case.total_k)


class Row:
    """Oracle results for one query row, computed from host copies of just what it needs."""

    def __init__(self, case, d, t, layers=(0,)):
        rows = DI.query_rows(case)
        _, b, p, base = rows[t]
        self.t, self.p, self.base = t, p, base
        kI = host64(d["k_idx"][base:base + p + 1])
        self.scores = O.indexer_scores_row(host64(d["q_idx"][t]), kI, host64(d["w"][t]))
        self.idx = O.topk_row(self.scores, case.index_topk)
        sel = self.idx[self.idx >= 0]
        self.attn = {}
        for l in layers:
            kv_rows = host64(d["kv"][l][base + torch.as_tensor(sel, device=d["kv"][l].device)])
            self.attn[l] = O.sparse_attention_row(host64(d["q"][l][t]), kv_rows, case.d_v,
                                                  case.softmax_scale)


def check_rows(case, d, scores, idx, outs, lses, sample, layers=(0,)):
    """Bit-exact scores and indices, and the attention bar applied to every query (and layer)
    on its own, for the sampled rows. Returns the per-row outputs and oracle outputs."""
    got_o = {l: [] for l in layers}
    ref_o = {l: [] for l in layers}
    worst = {l: (0.0, 0.0) for l in layers}
    for t in sample:
        r = Row(case, d, t, layers)
        n = r.p + 1
        if scores is not None:
            gs = scores[t, :n].double().cpu().numpy()
            bad = np.nonzero(gs != r.scores)[0]
            assert bad.size == 0, f"row {t}: {bad.size} score mismatches, first at {bad[:5]}"
        gi = idx[t].cpu().numpy().astype(np.int64)
        assert np.array_equal(gi, r.idx), f"row {t}: indices differ ({np.sum(gi != r.idx)})"
        for l in layers:
            g = outs[l][t].float().cpu().numpy()
            ok, a, rel = attn_close(g, r.attn[l][0])
            assert ok, f"row {t} layer {l}: max|d|={a:.3e} rel={rel:.3e}"
            worst[l] = (max(worst[l][0], a), max(worst[l][1], rel))
            got_o[l].append(g)
            ref_o[l].append(r.attn[l][0])
            if lses is not None:
                gl = lses[l][t].double().cpu().numpy()
                assert np.allclose(gl, r.attn[l][1], rtol=0, atol=2e-3), (t, gl[:4], r.attn[l][1][:4])
    for l in layers:
        say(f"  layer {l}: worst query max|d|={worst[l][0]:.3e} rel={worst[l][1]:.3e} "
            f"over {len(sample)} rows")
    return got_o, ref_o


def failing_queries(got, ref):
    """Queries (rows of got / ref) that miss the attention bar on their own."""
    return [i for i in range(len(got)) if not attn_close(got[i], ref[i])[0]]


def topk_all_rows_from_scores(case, scores, idx, threads=16):
    """Every row's indices against the oracle's top-k of that row's scores as the GPU computed
    them (the scores themselves are compared bit for bit with the oracle on sampled rows)."""
    from concurrent.futures import ThreadPoolExecutor
    rows = DI.query_rows(case)
    T = len(rows)
    chunk = 256
    for c0 in range(0, T, chunk):
        c1 = min(T, c0 + chunk)
        n_max = max(r[2] for r in rows[c0:c1]) + 1
        sc = scores[c0:c1, :n_max].double().cpu().numpy()
        gi = idx[c0:c1].cpu().numpy().astype(np.int64)

        def one(i):
            p = rows[c0 + i][2]
            return np.array_equal(gi[i], O.topk_row(sc[i, :p + 1], case.index_topk))

        with ThreadPoolExecutor(threads) as ex:
            ok = list(ex.map(one, range(c1 - c0)))
        bad = [c0 + i for i, v in enumerate(ok) if not v]
        assert not bad, f"rows {bad[:8]}: indices differ from the oracle's top-k of their scores"


def row_properties(case, idx):
    """Every row: ascending, unique, within 0..p, -1 only as trailing padding, and dense when
    p+1 <= k."""
    rows = DI.query_rows(case)
    k = case.index_topk
    p = torch.tensor([r[2] for r in rows], device=idx.device, dtype=torch.int64)
    i64 = idx.to(torch.int64)
    n_valid = torch.clamp(p + 1, max=k)
    pos = torch.arange(k, device=idx.device)[None, :]
    valid = pos < n_valid[:, None]
    assert bool(((i64 >= 0) == valid).all()), "padding not exactly where expected"
    assert bool((i64[valid.expand_as(i64)] >= 0).all())
    assert bool(((i64 <= p[:, None]) | ~valid).all()), "index beyond the causal position"
    inc = (i64[:, 1:] > i64[:, :-1]) | ~valid[:, 1:]
    assert bool(inc.all()), "not strictly ascending"
    dense = (p + 1) <= k
    if bool(dense.any()):
        want = torch.where(valid, pos.expand_as(i64), torch.full_like(i64, -1))
        assert bool((i64[dense] == want[dense]).all()), "dense rows must select 0..p"


def run_path(case, d, batch, layer=0, lse=True):
    scores = dsa.indexer_scores(d["q_idx"], d["k_idx"], d["w"], batch)
    idx = dsa.topk(scores, batch, case.index_topk)
    out, l = dsa.sparse_mla_fwd(d["q"][layer], d["kv"][layer], idx, batch, case.softmax_scale,
                                case.d_v, return_lse=lse)
    torch.cuda.synchronize()
    return scores, idx, out, l


# ------------------------------------------------------------------------------ workloads
def test_tiny_prefill_fp32_all_rows():
    case = DI.CASES["tiny_prefill_fp32"]
    say("case", case.name)
    d = DI.make_inputs(case, "cuda")
    batch = batch_of(case, d)
    scores, idx, out, lse = run_path(case, d, batch)
    row_properties(case, idx)
    got, ref = check_rows(case, d, scores, idx, {0: out}, {0: lse}, range(case.total_q))
    a, _ = attn_errors(np.stack(got[0]), np.stack(ref[0]))
    assert a < 1e-4, f"fp32 path should agree to ~1e-5, got {a}"


def test_decode_b32_l16k_all_rows():
    case = DI.CASES["decode_b32_l16k"]
    say("case", case.name)
    d = DI.make_inputs(case, "cuda")
    batch = batch_of(case, d)
    scores, idx, out, lse = run_path(case, d, batch)
    row_properties(case, idx)
    check_rows(case, d, scores, idx, {0: out}, {0: lse}, range(case.total_q))


@pytest.mark.parametrize("name", ["mtp_b32_l16k_q4", "mtp_b32_l16k_q4_shared"])
def test_mtp_decode_all_rows(name):
    """Four new tokens per sequence (one key stream scored for all four, in the indexer): every
    row against the oracle, through the separate calls and through dsa_forward (top-k inside
    the sparse-MLA launch)."""
    case = DI.CASES[name]
    say("case", case.name)
    d = DI.make_inputs(case, "cuda")
    batch = batch_of(case, d)
    scores, idx, out, lse = run_path(case, d, batch)
    row_properties(case, idx)
    check_rows(case, d, scores, idx, {0: out}, {0: lse}, range(case.total_q))
    o2, l2, i2 = dsa.forward(d["q"][0], d["kv"][0], batch, case.index_topk, case.softmax_scale,
                             case.d_v, q_idx=d["q_idx"], k_idx=d["k_idx"], w=d["w"])
    torch.cuda.synchronize()
    assert torch.equal(i2, idx)
    assert torch.equal(o2, out) and torch.equal(l2, lse)


def test_decode_forward_matches_separate_calls():
    case = DI.CASES["decode_b32_l16k"]
    d = DI.make_inputs(case, "cuda")
    batch = batch_of(case, d)
    s1, i1, o1, l1 = run_path(case, d, batch)
    o2, l2, i2 = dsa.forward(d["q"][0], d["kv"][0], batch, case.index_topk, case.softmax_scale,
                             case.d_v, q_idx=d["q_idx"], k_idx=d["k_idx"], w=d["w"])
    torch.cuda.synchronize()
    assert torch.equal(i1, i2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # determinism: a second run is bit-identical
    o3, l3, i3 = dsa.forward(d["q"][0], d["kv"][0], batch, case.index_topk, case.softmax_scale,
                             case.d_v, q_idx=d["q_idx"], k_idx=d["k_idx"], w=d["w"])
    torch.cuda.synchronize()
    assert torch.equal(i1, i3) and torch.equal(o1, o3) and torch.equal(l1, l3)


def test_forward_reuse_with_the_attention_workspace_only():
    """compute_indices = 0 reads the cached indices and needs only the sparse-MLA part of the
    forward workspace (placed at its start): a workspace of exactly that size, through the C
    ABI, gives the separate sparse-MLA call's output bit for bit."""
    import ctypes
    case = DI.CASES["decode_b32_l16k"]
    d = DI.make_inputs(case, "cuda")
    batch = batch_of(case, d)
    _, idx, o1, l1 = run_path(case, d, batch)
    L = dsa.lib()
    T, H = case.total_q, case.n_heads
    n_mla = dsa.workspace_size(dsa.OP_SPARSE_MLA, batch, case.index_topk, H, case.d_v)
    assert 0 < n_mla < dsa.workspace_size(dsa.OP_FORWARD, batch, case.index_topk, H, case.d_v)
    ws = torch.empty(n_mla, dtype=torch.uint8, device="cuda")
    out = torch.empty((T, H, case.d_v), dtype=case.dtype, device="cuda")
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    args = dsa._CForwardArgs(None, None, None, case.index_n_heads, case.index_head_dim,
                             case.index_topk, d["q"][0].data_ptr(), d["kv"][0].data_ptr(), H,
                             case.d_qk, case.d_v, case.softmax_scale, 1)
    sp = torch.cuda.current_stream().cuda_stream
    st = L.dsa_forward(batch.ptr, ctypes.byref(args), idx.data_ptr(), 0, out.data_ptr(),
                       lse.data_ptr(), ws.data_ptr(), n_mla, sp)
    assert st == 0, st
    # one byte short is refused before anything is launched
    st = L.dsa_forward(batch.ptr, ctypes.byref(args), idx.data_ptr(), 0, out.data_ptr(),
                       lse.data_ptr(), ws.data_ptr(), n_mla - 1, sp)
    assert st == 3, st
    torch.cuda.synchronize()
    assert torch.equal(o1, out) and torch.equal(l1, lse)


def test_multi_query_decode_full_size():
    """Two to four new query tokens per sequence (speculative / multi-token decode) at the
    decode sizes: 16 sequences of 16384 tokens, top-2048, 64 heads; every row checked."""
    nq = (2, 3, 4, 2, 3, 4, 2, 3, 4, 2, 3, 4, 2, 3, 4, 2)
    case = _small_case("mtp_b16_l16k", (16384,) * 16, nq)
    say("case", case.name)
    d = DI.make_inputs(case, "cuda")
    batch = batch_of(case, d)
    scores, idx, out, lse = run_path(case, d, batch)
    row_properties(case, idx)
    check_rows(case, d, scores, idx, {0: out}, {0: lse}, range(case.total_q))


def test_graph_capture_replays_match_eager():
    """The three calls captured in one HIP graph: every replay, with eager work and
    synchronisations between the replays, reproduces the eager results bit for bit (the calls
    allocate nothing and record no memset, so a captured step is the eager step)."""
    case = _small_case("graph_b8_l9000", (9000, 3000, 16384, 2500, 700, 12000, 5000, 2049),
                       (1,) * 8)
    d = DI.make_inputs(case, "cuda")
    batch = batch_of(case, d)
    T, ld = case.total_q, batch.max_seqlen_k
    scores = torch.zeros((T, ld), dtype=torch.float32, device="cuda")
    idx = torch.zeros((T, case.index_topk), dtype=torch.int32, device="cuda")
    out = torch.zeros((T, case.n_heads, case.d_v), dtype=case.dtype, device="cuda")
    lse = torch.zeros((T, case.n_heads), dtype=torch.float32, device="cuda")
    wsn = dsa.workspace_size(dsa.OP_SPARSE_MLA, batch, case.index_topk, case.n_heads, case.d_v)
    ws = torch.zeros(max(wsn, 1), dtype=torch.uint8, device="cuda")
    L = dsa.lib()

    def step(stream):
        sp = stream.cuda_stream
        st = L.dsa_indexer_scores(batch.ptr, d["q_idx"].data_ptr(), d["k_idx"].data_ptr(),
                                  d["w"].data_ptr(), case.index_n_heads, case.index_head_dim,
                                  1, scores.data_ptr(), ld, sp)
        st |= L.dsa_topk(batch.ptr, scores.data_ptr(), ld, case.index_topk, idx.data_ptr(),
                         None, 0, sp)
        st |= L.dsa_sparse_mla_fwd(batch.ptr, d["q"][0].data_ptr(), d["kv"][0].data_ptr(),
                                   idx.data_ptr(), case.index_topk, case.n_heads, case.d_qk,
                                   case.d_v, case.softmax_scale, 1, out.data_ptr(),
                                   lse.data_ptr(), ws.data_ptr(), ws.numel(), sp)
        assert st == 0, st

    step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref = [t.clone() for t in (scores, idx, out, lse)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(torch.cuda.current_stream())
    for rep in range(4):
        for t in (scores, idx, out, lse):
            t.zero_()                            # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("scores", "indices", "out", "lse"), (scores, idx, out, lse), ref):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager step"
    row_properties(case, idx)
    check_rows(case, d, scores, idx, {0: out}, {0: lse}, range(T))


@pytest.mark.slow
def test_prefill_chunk8k_l64k_all_rows():
    """Every one of the 8192 rows: indices equal the oracle's top-k of the row's scores; 264
    rows spread over the chunk (both ends, every 32nd row): scores bit-exact against the
    oracle's indexer and the attention bar per query."""
    case = DI.CASES["prefill_chunk8k_l64k"]
    say("case", case.name)
    d = DI.make_inputs(case, "cuda")
    batch = batch_of(case, d)
    scores, idx, out, lse = run_path(case, d, batch)
    row_properties(case, idx)
    T = case.total_q
    topk_all_rows_from_scores(case, scores, idx)
    say("  top-k: all rows equal the oracle's selection from their scores")
    sample = sorted(set([0, 1, 15, 16, 17, 777, 4095, 4096, T - 17, T - 2, T - 1] +
                        list(range(5, T, 32))))
    assert len(sample) >= 256
    check_rows(case, d, scores, idx, {0: out}, {0: lse}, sample)


@pytest.mark.slow
def test_indexshare_b8_l256k_all_rows():
    """One index pass shared by 4 layers: every row's scores and indices against the oracle,
    every layer's output per query; reuse is bit-identical to separate calls."""
    case = DI.CASES["indexshare_b8_l256k"]
    say("case", case.name)
    d = DI.make_inputs(case, "cuda")
    batch = batch_of(case, d)
    shared = None
    outs, lses = {}, {}
    for l in range(case.layers):
        o, ls, shared = dsa.forward(d["q"][l], d["kv"][l], batch, case.index_topk,
                                    case.softmax_scale, case.d_v, q_idx=d["q_idx"],
                                    k_idx=d["k_idx"], w=d["w"], shared_indices=shared,
                                    compute_indices=(l == 0))
        outs[l], lses[l] = o, ls
    torch.cuda.synchronize()
    row_properties(case, shared)
    # reuse is bit-identical to running the layer on its own with the same indices
    for l in (1, 3):
        o, ls = dsa.sparse_mla_fwd(d["q"][l], d["kv"][l], shared, batch, case.softmax_scale,
                                   case.d_v)
        torch.cuda.synchronize()
        assert torch.equal(o, outs[l]) and torch.equal(ls, lses[l])
    # the cached indices are what a fresh indexer + top-k produce
    scores = dsa.indexer_scores(d["q_idx"], d["k_idx"], d["w"], batch)
    fresh = dsa.topk(scores, batch, case.index_topk)
    torch.cuda.synchronize()
    assert torch.equal(fresh, shared)
    check_rows(case, d, scores, shared, outs, lses, range(case.total_q),
               layers=tuple(range(case.layers)))


@pytest.mark.slow
def test_mixed_b16_l512_1m_all_rows():
    """Sixteen sequences of 512..1048576 tokens (four take the dense path): every row's scores,
    indices and output against the oracle."""
    case = DI.CASES["mixed_b16_l512_1m"]
    say("case", case.name)
    d = DI.make_inputs(case, "cuda")
    batch = batch_of(case, d)
    scores, idx, out, lse = run_path(case, d, batch)
    row_properties(case, idx)
    check_rows(case, d, scores, idx, {0: out}, {0: lse}, range(case.total_q))


# ----------------------------------------------------------------------------- edge cases
def _small_case(name, seqlens_k, seqlens_q, **kw):
    return DI.custom_case(name, seqlens_k, seqlens_q,
                          seed_base=zlib.crc32(name.encode()) % 100000 * 100, **kw)


@pytest.mark.parametrize("lens,nq,k", [
    ((1,), (1,), 2048),                       # single visible token
    ((2047, 2048, 2049, 2050), (1, 1, 1, 1), 2048),   # around the dense threshold
    ((37, 3000, 5, 9000, 65), (1, 2, 1, 3, 4), 64),   # ragged decode + multi-query rows
    ((300, 129), (40, 17), 64),              # short prefill chunks (prefill indexer kernel)
    ((4100,), (4100,), 2048),                # whole-sequence prefill
    ((9000,), (1,), 4096),                   # one query, 32 splits of two tiles each
    ((5000, 7000), (1, 1), 3000),            # k not a multiple of the 64-row tile, 24 splits
    # several new tokens per sequence on one key stream: groups of four, a partial last group
    ((9000, 7, 3000, 20000, 12), (7, 7, 5, 15, 1), 2048),
    ((2050, 4, 6000), (4, 4, 3), 2048),       # tokens near the dense threshold, nq == L
])
def test_ragged_edge_cases(lens, nq, k):
    case = _small_case(f"edge_{lens}_{nq}_{k}", lens, nq, index_topk=k)
    say("case", case.name)
    d = DI.make_inputs(case, "cuda")
    batch = batch_of(case, d)
    dsa.check_batch(batch)
    scores, idx, out, lse = run_path(case, d, batch)
    row_properties(case, idx)
    T = case.total_q
    sample = range(T) if T <= 64 else sorted(set([0, 1, T // 2, T - 2, T - 1] + list(range(0, T, T // 16))))
    check_rows(case, d, scores, idx, {0: out}, {0: lse}, sample)


def test_index_heads_64_and_attention_heads_128():
    case = _small_case("heads", (5000, 700), (1, 1), index_n_heads=64, n_heads=128)
    d = DI.make_inputs(case, "cuda")
    batch = batch_of(case, d)
    scores, idx, out, lse = run_path(case, d, batch)
    check_rows(case, d, scores, idx, {0: out}, {0: lse}, range(case.total_q))


@pytest.mark.parametrize("heads", [32, 96])
def test_attention_heads_odd_number_of_32_head_groups(heads):
    """The last 64-head workgroup has an empty upper half (it computes on other heads' queries
    and writes nothing); split and single-split launches."""
    case = _small_case(f"heads{heads}", (5000, 700, 3100), (1, 1, 2), n_heads=heads)
    d = DI.make_inputs(case, "cuda")
    batch = batch_of(case, d)
    scores, idx, out, lse = run_path(case, d, batch)
    assert out.shape[1] == heads
    check_rows(case, d, scores, idx, {0: out}, {0: lse}, range(case.total_q))


def test_all_equal_scores_take_lowest_positions():
    case = _small_case("ties", (9000, 3000), (1, 2))
    d = DI.make_inputs(case, "cuda")
    d["w"].zero_()                              # every score is 0 (some -0.0 via (-x)*0)
    d["q_idx"][:, :, ::2] *= -1
    batch = batch_of(case, d)
    scores = dsa.indexer_scores(d["q_idx"], d["k_idx"], d["w"], batch)
    idx = dsa.topk(scores, batch, case.index_topk)
    torch.cuda.synchronize()
    want = torch.arange(case.index_topk, device="cuda", dtype=torch.int32)
    assert bool((idx == want[None, :]).all())


def test_heavy_ties_match_oracle():
    # w in {0, 1} and q_I in {-1, 0, 1}: scores take few values, so the k-th falls in a big tie
    case = _small_case("heavy_ties", (20000, 40000), (1, 1), idx_range=1, w_range=1)
    d = DI.make_inputs(case, "cuda")
    d["w"].clamp_(min=0)
    batch = batch_of(case, d)
    scores, idx, out, lse = run_path(case, d, batch)
    check_rows(case, d, scores, idx, {0: out}, {0: lse}, range(case.total_q))


def test_sparse_mla_invariants():
    case = _small_case("mla_inv", (6000, 2500, 9000), (1, 1, 1))
    d = DI.make_inputs(case, "cuda")
    batch = batch_of(case, d)
    scores, idx, out, lse = run_path(case, d, batch)
    # permuting each row's selected set leaves the output unchanged (within tolerance)
    g = torch.Generator(device="cuda").manual_seed(7)
    perm = torch.argsort(torch.rand(idx.shape, generator=g, device="cuda"), dim=1)
    out_p, lse_p = dsa.sparse_mla_fwd(d["q"][0], d["kv"][0], torch.gather(idx, 1, perm).contiguous(),
                                      batch, case.softmax_scale, case.d_v)
    torch.cuda.synchronize()
    for t in range(case.total_q):
        ok, a, r = attn_close(out_p[t].float().cpu().numpy(), out[t].float().cpu().numpy(),
                              1e-2, 5e-3)
        assert ok, (t, a, r)
    # V == 1 gives 1 everywhere
    kv1 = d["kv"][0].clone()
    kv1[:, :case.d_v] = 1
    o1, _ = dsa.sparse_mla_fwd(d["q"][0], kv1, idx, batch, case.softmax_scale, case.d_v)
    torch.cuda.synchronize()
    assert bool((o1.float() == 1).all())
    # -1 and out-of-range entries are skipped: masking half the row equals dropping it
    half = idx.clone()
    half[:, 1::2] = -1
    oh, lh = dsa.sparse_mla_fwd(d["q"][0], d["kv"][0], half, batch, case.softmax_scale, case.d_v)
    oor = idx.clone()
    oor[:, 1::2] = 10 ** 8
    oo, lo = dsa.sparse_mla_fwd(d["q"][0], d["kv"][0], oor, batch, case.softmax_scale, case.d_v)
    torch.cuda.synchronize()
    assert torch.equal(oh, oo) and torch.equal(lh, lo)
    for t in range(case.total_q):
        r = Row(case, d, t)
        sel = half[t].cpu().numpy()
        sel = sel[sel >= 0]
        o_ref, _ = O.sparse_attention_row(host64(d["q"][0][t]),
                                          host64(d["kv"][0][r.base + torch.as_tensor(sel, device="cuda")]),
                                          case.d_v, case.softmax_scale)
        ok, a, rel = attn_close(oh[t].float().cpu().numpy(), o_ref)
        assert ok, (t, a, rel)
    # a row with no valid index gives zeros and lse = -inf
    none = torch.full_like(idx, -1)
    on, ln = dsa.sparse_mla_fwd(d["q"][0], d["kv"][0], none, batch, case.softmax_scale, case.d_v)
    torch.cuda.synchronize()
    assert bool((on.float() == 0).all()) and bool(torch.isneginf(ln).all())


def _control_ref(case, d, r, name):
    """The oracle's output for row r with one planted mistake in the reference."""
    q = host64(d["q"][0][r.t])
    sel = r.idx[r.idx >= 0].copy()
    scale = case.softmax_scale
    if name == "one_wrong_index":
        unsel = np.setdiff1d(np.arange(r.p + 1), sel)
        sel[len(sel) // 2] = unsel[0]
    kvr = host64(d["kv"][0][r.base + torch.as_tensor(np.sort(sel), device="cuda")])
    if name == "dropped_rope":
        kvr[:, case.d_v:] = 0
    if name == "scale_1/sqrt(512)":
        scale = 1 / math.sqrt(512)
    return O.sparse_attention_row(q, kvr, case.d_v, scale)[0]


def _controls(case, d, out, rows, which, victims=None):
    """Each control plants a mistake in the reference of the queries in `victims` (all rows by
    default) and must make exactly those queries fail the per-query bar."""
    got = [out[r.t].float().cpu().numpy() for r in rows]
    good = [r.attn[0][0] for r in rows]
    assert failing_queries(got, good) == []
    victims = list(range(len(rows))) if victims is None else list(victims)
    res = {}
    for name in which:
        ref = [(_control_ref(case, d, r, name) if i in victims else good[i])
               for i, r in enumerate(rows)]
        fails = failing_queries(got, ref)
        pooled_ok, pa, prel = attn_close(np.stack(got), np.stack(ref))
        say(f"  negative control {name} on {len(victims)} of {len(rows)} queries: failing "
            f"{fails}; pooled over the queries the bar would read max|d|={pa:.3e} "
            f"rel={prel:.3e} ({'pass' if pooled_ok else 'fail'})")
        res[name] = fails == victims
    return res


def test_negative_controls_decode():
    """At the decode distribution (q, kv ~ 0.1 N(0,1), scale 1/24) the logits are nearly flat,
    so the output is essentially the mean value row of the selected set. The bar applies to each
    query on its own: one wrong row in one query of the 32 must fail that query (pooled over all
    32 queries the same error would pass), and one wrong row in every query fails each."""
    case = DI.CASES["decode_b32_l16k"]
    d = DI.make_inputs(case, "cuda")
    batch = batch_of(case, d)
    scores, idx, out, lse = run_path(case, d, batch)
    rows = [Row(case, d, t) for t in range(case.total_q)]
    res = _controls(case, d, out, rows, ["one_wrong_index"], victims=[5])
    assert all(res.values()), res
    res = _controls(case, d, out, rows[:8], ["one_wrong_index"])
    assert all(res.values()), res


def test_unit_variance_decode_and_controls():
    """q, kv ~ N(0,1): logits have unit spread, so the QK product matters; parity on every row and
    the bar must catch dropped rope columns, a wrong scale and one wrong index in any query."""
    case = _small_case("decode_sigma1", (16384,) * 8, (1,) * 8, sigma=1.0)
    d = DI.make_inputs(case, "cuda")
    batch = batch_of(case, d)
    scores, idx, out, lse = run_path(case, d, batch)
    check_rows(case, d, scores, idx, {0: out}, {0: lse}, range(case.total_q))
    rows = [Row(case, d, t) for t in range(case.total_q)]
    res = _controls(case, d, out, rows, ["one_wrong_index", "dropped_rope", "scale_1/sqrt(512)"])
    assert all(res.values()), res
    res = _controls(case, d, out, rows, ["one_wrong_index"], victims=[3])
    assert all(res.values()), res


def _crafted_topk(rows_scores, k):
    """Run dsa_topk on explicit score rows (one decode sequence per row) and compare with the
    oracle's top-k row by row."""
    lens = [len(r) for r in rows_scores]
    batch = dsa.Batch.from_lengths([1] * len(lens), lens)
    ld = max(lens)
    sc = torch.zeros((len(lens), ld), dtype=torch.float32)
    for i, r in enumerate(rows_scores):
        sc[i, :len(r)] = torch.from_numpy(np.asarray(r, dtype=np.float32))
    idx = dsa.topk(sc.cuda(), batch, k)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    for i, r in enumerate(rows_scores):
        want = O.topk_row(np.asarray(r, dtype=np.float32).astype(np.float64), k)
        assert np.array_equal(got[i], want), (i, len(r), np.sum(got[i] != want))


def _crafted_topk_at(rows_scores, k, shift):
    """As _crafted_topk, with every row of length ld = the longest row, the score matrix starting
    `shift` floats into its buffer and ending where the buffer ends."""
    lens = [len(r) for r in rows_scores]
    batch = dsa.Batch.from_lengths([1] * len(lens), lens)
    T, ld = len(lens), max(lens)
    buf = torch.zeros(shift + T * ld, dtype=torch.float32)
    sc = buf[shift:].view(T, ld)
    for i, r in enumerate(rows_scores):
        sc[i, :len(r)] = torch.from_numpy(np.asarray(r, dtype=np.float32))
    gbuf = buf.cuda()
    idx = dsa.topk(gbuf[shift:].view(T, ld), batch, k)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    for i, r in enumerate(rows_scores):
        want = O.topk_row(np.asarray(r, dtype=np.float32).astype(np.float64), k)
        assert np.array_equal(got[i], want), (i, len(r), np.sum(got[i] != want))


@pytest.mark.parametrize("shift", [1, 3])
def test_topk_unaligned_rows_to_the_buffer_end(shift):
    """Score rows that start off a 16-byte boundary (odd row length, matrix offset into its
    buffer) and are visible to their last position: each row's first and last 16-byte groups
    straddle the row's ends and are read element by element, so no read leaves the buffer. The
    oracle's top-k on the split-row path (8 rows of 40001), the register path (80 rows of 20001)
    and the streamed path (70 rows of 70001)."""
    rng = np.random.default_rng(40 + shift)
    for T, L in ((8, 40001), (80, 20001), (70, 70001)):
        rows = [rng.integers(-50, 51, L).astype(np.float32) for _ in range(T)]
        rows[1] = rng.normal(size=L).astype(np.float32)
        rows[-1][-3:] = 1000.0                     # the last row's last positions are selected
        _crafted_topk_at(rows, 2048, shift)


def test_topk_crafted_rows():
    rng = np.random.default_rng(5)
    rows = []
    z = rng.integers(-1, 2, 50000).astype(np.float32)          # heavy ties incl. signed zeros
    z[(z == 0) & (rng.random(50000) < 0.5)] = -0.0
    rows.append(z)
    rows.append(np.where(rng.random(40000) < 0.5, np.float32(0.0), np.float32(-0.0)))
    rows.append(rng.normal(size=70000).astype(np.float32))      # longer than the LDS key cache
    rows.append(rng.normal(size=9000).astype(np.float32) * 1e-30)   # tiny magnitudes
    rows.append(np.concatenate([np.full(3000, 5.0), np.full(3000, -5.0)]).astype(np.float32))
    rows.append(np.arange(20000, dtype=np.float32))             # strictly increasing
    rows.append(-np.arange(20000, dtype=np.float32))            # strictly decreasing
    big = rng.integers(-3, 4, 300000).astype(np.float32)        # long row, huge tie groups
    rows.append(big)
    rows.append(np.array([np.inf, -np.inf, 1.0, 3.0e38, -3.0e38] * 1000, dtype=np.float32))
    # one outlier stretches the linear bins so far that both linear rounds put every other
    # score into one fine bin: the threshold is found among the listed candidates
    out = (1.0 + rng.random(100000) * 1e-3).astype(np.float32)
    out[77777] = 1e30
    rows.append(out)
    # candidates with large tie groups straddling the k-th score
    tie = np.round(rng.random(90000) * 50).astype(np.float32) * np.float32(1e-6) + np.float32(1.0)
    tie[12345] = -1e30
    rows.append(tie)
    _crafted_topk(rows, 2048)
    _crafted_topk([r[:5000] for r in rows], 7)


def _few_bin_row(rng, n_bin):
    """A row whose k-th largest score (k = 2048) lies in a linear round-0 bin holding n_bin
    scores with ties: the range [0, 2048] gives bins of width 1, 2000 distinct scores sit in
    bins 1000..1999, the bin [500, 501) holds n_bin scores in three tie groups, and 6000
    scores lie below it, in shuffled positions."""
    hi = 1000.0 + 0.5 * np.arange(2000)
    groups = [500.75] * 34 + [500.5] * 20 + [500.25] * 10 + [500.125] * (n_bin - 64)
    lo = rng.random(6000) * 499.0
    row = np.concatenate([hi, groups, lo, [0.0, 2048.0]]).astype(np.float32)
    return row[rng.permutation(row.shape[0])]


def test_topk_few_scores_in_the_threshold_bin():
    """64 scores in the threshold's round-0 bin are ranked directly; 65 take the second
    histogram round. Both must match the oracle, ties going to the lowest positions."""
    rng = np.random.default_rng(21)
    rows = [_few_bin_row(rng, 64), _few_bin_row(rng, 65), _few_bin_row(rng, 64)[:5000]]
    _crafted_topk(rows, 2048)


def test_topk_many_long_rows():
    """More rows than the split-row path takes: one workgroup per row, the row in chunks."""
    rng = np.random.default_rng(9)
    rows = [rng.integers(-6, 7, int(n)).astype(np.float32)
            for n in rng.integers(33000, 70000, 72)]
    rows[3] = rng.normal(size=rows[3].shape[0]).astype(np.float32)
    _crafted_topk(rows, 2048)


def test_topk_streamed_rows_two_workgroups_per_cu():
    """At least 512 streamed rows (longer than one register chunk, k within the candidate buffer):
    512-thread workgroups, two per CU, each row in chunks of 16384 positions, with ties and a
    row shorter than one chunk among them."""
    rng = np.random.default_rng(12)
    lens = rng.integers(33000, 41000, 520)
    rows = [rng.integers(-6, 7, int(n)).astype(np.float32) for n in lens]
    rows[7] = rng.normal(size=rows[7].shape[0]).astype(np.float32)
    rows[100] = np.full(int(lens[100]), 2.0, dtype=np.float32)       # one tie group
    rows[200] = rows[200][:9000]                                       # one chunk
    _crafted_topk(rows, 2048)


def test_topk_many_long_rows_large_k():
    """Rows longer than one register chunk with k above the candidate buffer: every pass
    re-reads the row chunk by chunk."""
    rng = np.random.default_rng(11)
    rows = [rng.integers(-5, 6, int(n)).astype(np.float32)
            for n in rng.integers(33000, 45000, 66)]
    rows[5] = rng.normal(size=rows[5].shape[0]).astype(np.float32)
    _crafted_topk(rows, 3000)


def test_topk_split_rows_mixed_lengths():
    """A few long rows with short and dense rows beside them (the split-row path)."""
    rng = np.random.default_rng(10)
    lens = [1000, 2048, 2049, 8191, 8192, 8193, 40000, 131075, 300001]
    rows = [rng.normal(size=n).astype(np.float32) for n in lens]
    rows[7] = rng.integers(-4, 5, lens[7]).astype(np.float32)
    _crafted_topk(rows, 2048)
    _crafted_topk(rows, 6000)


def test_topk_split_rows_beyond_one_launch():
    """Rows of more than 256 chunks of 8192 positions take the five-launch split path (the
    one-launch path, whose row barriers need every chunk of a row resident, takes every shorter
    row): a row of 2,200,001 positions in 41 tie groups, one of 2,097,153 normal scores just past
    the bound, and a short row beside them."""
    rng = np.random.default_rng(13)
    rows = [rng.integers(-20, 21, 2_200_001).astype(np.float32),
            rng.normal(size=2_097_153).astype(np.float32),
            rng.normal(size=50000).astype(np.float32)]
    _crafted_topk(rows, 2048)


def test_split_topk_on_a_garbage_workspace(monkeypatch):
    """The one-launch split top-k zero-fills its row state before use: with every workspace
    filled with 0xAB bytes, dsa_topk (its own clear launch) and dsa_forward (the decode indexer
    clears the state on the side), each called twice in a row, give the oracle's top-k of the
    GPU scores on every row, bit for bit, and dsa_forward's indices equal dsa_topk's."""
    orig = dsa._workspace

    def garbage(nbytes, device):
        t, n = orig(nbytes, device)
        if t is not None:
            t.fill_(0xAB)
        return t, n

    monkeypatch.setattr(dsa, "_workspace", garbage)
    case = _small_case("garbage_ws", (100000, 70001, 40000, 3000), (1, 1, 2, 1))
    say("case", case.name)
    d = DI.make_inputs(case, "cuda")
    batch = batch_of(case, d)
    scores = dsa.indexer_scores(d["q_idx"], d["k_idx"], d["w"], batch)
    for _ in range(2):
        idx = dsa.topk(scores, batch, case.index_topk)
        out, lse, fidx = dsa.forward(d["q"][0], d["kv"][0], batch, case.index_topk,
                                     case.softmax_scale, case.d_v, q_idx=d["q_idx"],
                                     k_idx=d["k_idx"], w=d["w"])
        torch.cuda.synchronize()
        sc = scores.cpu().numpy()
        got, fgot = idx.cpu().numpy(), fidx.cpu().numpy()
        for t, b, p, base in DI.query_rows(case):
            want = O.topk_row(sc[t, :p + 1].astype(np.float64), case.index_topk)
            assert np.array_equal(got[t], want), ("dsa_topk", t)
            assert np.array_equal(fgot[t], want), ("dsa_forward", t)


def test_reference_max_restart_path():
    """Rows whose logits exceed the first tile's maximum by far more than the softmax headroom
    force the attention kernel to raise its reference maxima and redo the split; the result must
    still match the oracle."""
    case = _small_case("restart", (6000, 9000, 3000), (1, 1, 1), sigma=1.0)
    d = DI.make_inputs(case, "cuda")
    batch = batch_of(case, d)
    scores = dsa.indexer_scores(d["q_idx"], d["k_idx"], d["w"], batch)
    idx = dsa.topk(scores, batch, case.index_topk)
    torch.cuda.synchronize()
    kv = d["kv"][0].clone()
    rows = DI.query_rows(case)
    for t, b, p, base in rows:
        sel = idx[t][idx[t] >= 0].long()
        late = sel[-3:]                                  # in the last tile of the last split
        kv[base + late] = (kv[base + late].float() * 40).to(kv.dtype)
    out, lse = dsa.sparse_mla_fwd(d["q"][0], kv, idx, batch, case.softmax_scale, case.d_v)
    torch.cuda.synchronize()
    got, ref = [], []
    for t, b, p, base in rows:
        sel = idx[t][idx[t] >= 0].cpu().numpy()
        o, l = O.sparse_attention_row(host64(d["q"][0][t]),
                                      host64(kv[base + torch.as_tensor(sel, device="cuda")]),
                                      case.d_v, case.softmax_scale)
        got.append(out[t].float().cpu().numpy())
        ref.append(o)
        assert np.allclose(lse[t].double().cpu().numpy(), l, rtol=1e-4, atol=1e-2)
    # value rows scaled by 40 make outputs ~100x the workload's, so max|d| is taken relative
    for i, (g, r) in enumerate(zip(got, ref)):
        ok, a, rel = attn_close(g, r, max_abs=2e-2 * np.abs(r).max())
        say(f"  restart path, query {i}: max|d|={a:.3e} (max|ref| {np.abs(r).max():.1f}) "
            f"rel={rel:.3e}")
        assert ok, (i, a, rel)


def test_split_partials_against_one_split():
    """The error the bf16 split partials add: one decode query attended once alone (16 splits of
    two tiles, partials in bf16 merged by mla_combine) and once as one of 256 identical queries
    of a batch (one split: no partials), both against the oracle and against each other."""
    L, k, H = 16384, 2048, 64
    kv = DI.normal((L, 576), 0.1, torch.bfloat16, "cuda", 9101)
    q1 = DI.normal((1, H, 576), 0.1, torch.bfloat16, "cuda", 9102)
    g = torch.Generator(device="cpu").manual_seed(9103)
    sel = torch.sort(torch.randperm(L - 256, generator=g)[:k]).values.to(torch.int32)
    scale = 1 / 24
    outs = {}
    for T in (1, 256):
        batch = dsa.Batch.from_lengths([T], [L], device="cuda")
        q = q1.expand(T, H, 576).contiguous()
        idx = sel.to("cuda")[None, :].expand(T, k).contiguous()
        out, lse = dsa.sparse_mla_fwd(q, kv, idx, batch, scale, 512)
        torch.cuda.synchronize()
        outs[T] = (out[0].float().cpu().numpy(), lse[0].float().cpu().numpy())
        if T == 256:   # every copy of the query got the same bits
            assert bool((out == out[0:1]).all())
    ref, ref_lse = O.sparse_attention_row(host64(q1[0]), host64(kv[sel.long().to("cuda")]), 512,
                                          scale)
    a16, r16 = attn_errors(outs[1][0], ref)
    a1, r1 = attn_errors(outs[256][0], ref)
    ad, rd = attn_errors(outs[1][0], outs[256][0])
    say(f"  16 splits vs oracle: max|d|={a16:.3e} rel={r16:.3e}; one split vs oracle: "
        f"max|d|={a1:.3e} rel={r1:.3e}; 16 vs 1 split: max|d|={ad:.3e} rel={rd:.3e}; "
        f"lse 16 vs 1 split max|d|={np.abs(outs[1][1] - outs[256][1]).max():.3e}")
    assert attn_close(outs[1][0], ref)[0] and attn_close(outs[256][0], ref)[0]
    assert np.allclose(outs[1][1], ref_lse, rtol=1e-4, atol=2e-3)


@pytest.mark.parametrize("lens,nq,kw", [
    ((16384,) * 32, (1,) * 32, {}),                                   # the decode workload shape
    ((1, 2047, 2048, 2049, 16384, 9000), (1, 1, 1, 1, 1, 1), {}),      # around the dense threshold
    ((5000, 16384, 3000, 12000), (2, 4, 1, 3), {}),                   # several queries per row
    ((16384, 9000, 7000), (1, 1, 1), {"idx_range": 1, "w_range": 1}),  # heavy ties
    ((9000, 16000), (1, 1), {"index_topk": 4096}),                    # 32 splits of two tiles
    ((5000, 7000, 16384), (1, 1, 1), {"index_topk": 3000}),           # k not a multiple of 64
    ((16384, 6000), (1, 2), {"n_heads": 128}),                         # two head groups per split
    ((16384, 6000, 3333), (1, 1, 1), {"n_heads": 32}),
    ((16385, 9000), (1, 1), {}),                   # one position past the in-launch bound
])
def test_forward_fused_selection_matches_topk(lens, nq, kw):
    """dsa_forward on rows of at most 16384 positions selects the top-k inside the sparse-MLA
    kernel: the shared indices must equal dsa_topk's on the same scores and the oracle's, and the
    outputs those of the separate sparse-MLA call, bit for bit."""
    case = _small_case(f"fused_{lens}_{nq}_{sorted(kw.items())}", lens, nq, **kw)
    d = DI.make_inputs(case, "cuda")
    batch = batch_of(case, d)
    o, l, shared = dsa.forward(d["q"][0], d["kv"][0], batch, case.index_topk, case.softmax_scale,
                               case.d_v, q_idx=d["q_idx"], k_idx=d["k_idx"], w=d["w"])
    scores = dsa.indexer_scores(d["q_idx"], d["k_idx"], d["w"], batch)
    idx = dsa.topk(scores, batch, case.index_topk)
    o2, l2 = dsa.sparse_mla_fwd(d["q"][0], d["kv"][0], idx, batch, case.softmax_scale, case.d_v)
    torch.cuda.synchronize()
    assert torch.equal(shared, idx)
    assert torch.equal(o, o2) and torch.equal(l, l2)
    rows = range(case.total_q) if case.total_q <= 12 else [0, 7, 19, case.total_q - 1]
    check_rows(case, d, scores, shared, {0: o}, {0: l}, rows)


def _order_keys(x):
    """Order-preserving uint32 keys of fp32 scores (-0.0 as +0.0), as the selection defines them."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).copy()
    u[u == 0x80000000] = 0
    neg = (u & 0x80000000) != 0
    return np.where(neg, ~u, u | 0x80000000).astype(np.uint32)


def test_forward_fused_selection_real_valued_scores():
    """Real-valued indexer weights: the threshold's 22-bit key prefix is then often shared by
    several distinct scores, so the in-launch selection needs its third radix round (integer
    scores never do). Indices must equal the oracle's top-k of the same scores on every row, and
    the outputs those of the separate calls; the test also checks on the CPU that some rows do
    take the third round."""
    case = _small_case("fused_real", (16384,) * 24 + (9000, 5000, 13000), (1,) * 27)
    d = DI.make_inputs(case, "cuda")
    g = torch.Generator(device="cuda").manual_seed(77)
    d["w"] = torch.randn(d["w"].shape, generator=g, device="cuda") * 0.37
    batch = batch_of(case, d)
    o, l, shared = dsa.forward(d["q"][0], d["kv"][0], batch, case.index_topk, case.softmax_scale,
                               case.d_v, q_idx=d["q_idx"], k_idx=d["k_idx"], w=d["w"])
    scores = dsa.indexer_scores(d["q_idx"], d["k_idx"], d["w"], batch)
    idx = dsa.topk(scores, batch, case.index_topk)
    o2, l2 = dsa.sparse_mla_fwd(d["q"][0], d["kv"][0], idx, batch, case.softmax_scale, case.d_v)
    torch.cuda.synchronize()
    assert torch.equal(shared, idx)
    assert torch.equal(o, o2) and torch.equal(l, l2)
    topk_all_rows_from_scores(case, scores, shared)
    third = 0
    for t, _, p, _ in DI.query_rows(case):
        keys = _order_keys(scores[t, :p + 1].cpu().numpy())
        if p + 1 <= case.index_topk:
            continue
        thr = np.sort(keys)[::-1][case.index_topk - 1]
        third += np.unique(keys[(keys >> 10) == (thr >> 10)]).size > 1
    say(f"  rows needing the third round: {third} of {case.total_q}")
    assert third > 0


def test_forward_fused_selection_equal_scores():
    """Every score equal (zero weights; signed zeros among them): the fused selection takes the
    lowest positions, like dsa_topk."""
    case = _small_case("fused_ties", (9000, 16384, 3000), (1, 2, 1))
    d = DI.make_inputs(case, "cuda")
    d["w"].zero_()
    d["q_idx"][:, :, ::2] *= -1
    batch = batch_of(case, d)
    _, _, shared = dsa.forward(d["q"][0], d["kv"][0], batch, case.index_topk, case.softmax_scale,
                               case.d_v, q_idx=d["q_idx"], k_idx=d["k_idx"], w=d["w"])
    torch.cuda.synchronize()
    want = torch.arange(case.index_topk, device="cuda", dtype=torch.int32)
    assert bool((shared == want[None, :]).all())

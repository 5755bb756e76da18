"""Seeded synthetic inputs for the DSA hot path (shared by the oracle tests, the GPU tests
and the benchmark).

This module draws random tensors and lays out ragged batches. It holds none of the
method's arithmetic: no scoring, selection or attention happens here.

Every tensor comes from its own torch generator seeded with ``1000*case + tensor_id``
(ids: k_idx=1, q_idx=2, w=3, kv of layer l = 10+l, q of layer l = 20+l, the share mask of
correlated query tokens = 4). Integer-valued
tensors are drawn uniformly over the inclusive integer range and cast to the case dtype
(exact). Normal tensors are ``randn * sigma`` rounded once to the case dtype. Tensors are
generated on the requested device; the oracle always receives a host copy of exactly the
values the GPU sees.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np
import torch

ID_K_IDX, ID_Q_IDX, ID_W, ID_SHARE = 1, 2, 3, 4
ID_KV0, ID_Q0 = 10, 20


@dataclasses.dataclass(frozen=True)
class Case:
    """Shapes and value ranges of one synthetic workload."""
    name: str
    seed_base: int
    dtype: torch.dtype
    seqlens_k: tuple          # context length L_b of every sequence
    seqlens_q: tuple          # new query tokens nq_b of every sequence (nq_b <= L_b)
    index_n_heads: int        # H_I
    index_head_dim: int       # d_I
    idx_range: int            # q_I, k_I uniform integers in [-idx_range, idx_range]
    w_range: int              # w uniform integers in [-w_range, w_range]
    index_topk: int           # k
    n_heads: int              # H
    d_qk: int                 # latent + rope width
    d_v: int                  # value width (leading columns of the latent row)
    sigma: float              # q, kv ~ N(0, sigma^2)
    layers: int = 1           # sparse-MLA layers sharing one index pass
    q_share: float = 0.0      # later query tokens of a sequence copy this fraction of their
    #                           indexer entries (q_I, w) from the token before them

    @property
    def batch(self) -> int:
        return len(self.seqlens_k)

    @property
    def total_q(self) -> int:
        return int(sum(self.seqlens_q))

    @property
    def total_k(self) -> int:
        return int(sum(self.seqlens_k))

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.d_qk)


def mixed_lengths(seed: int = 5, n_draw: int = 14, lo: int = 512, hi: int = 1048576) -> List[int]:
    """Context lengths log-uniform in [lo, hi]: ``n_draw`` draws ``floor(exp(U(ln lo, ln hi)))``
    plus both endpoints, shuffled, all from ``numpy.random.default_rng(seed)``."""
    rng = np.random.default_rng(seed)
    u = rng.uniform(math.log(lo), math.log(hi), n_draw)
    lens = [lo, hi] + [int(math.floor(math.exp(x))) for x in u]
    return [int(x) for x in rng.permutation(np.array(lens, dtype=np.int64))]


_GLM_DIMS = dict(index_n_heads=32, index_head_dim=128, idx_range=4, w_range=2, index_topk=2048,
                 n_heads=64, d_qk=576, d_v=512, sigma=0.1)

CASES: Dict[str, Case] = {
    # tiny causal prefill in fp32: one sequence of 256 tokens attending to itself
    "tiny_prefill_fp32": Case("tiny_prefill_fp32", 1000, torch.float32, (256,), (256,),
                              index_n_heads=4, index_head_dim=32, idx_range=3, w_range=2,
                              index_topk=64, n_heads=8, d_qk=80, d_v=64, sigma=1.0),
    # decode: 32 sequences of 16384 tokens, one new query each
    "decode_b32_l16k": Case("decode_b32_l16k", 2000, torch.bfloat16, (16384,) * 32, (1,) * 32,
                            **_GLM_DIMS),
    # chunked prefill: 8192 new queries (positions 57344..65535) over a 65536-token cache
    "prefill_chunk8k_l64k": Case("prefill_chunk8k_l64k", 3000, torch.bfloat16, (65536,), (8192,),
                                 **_GLM_DIMS),
    # long-context decode, one index pass shared by 4 sparse-MLA layers
    "indexshare_b8_l256k": Case("indexshare_b8_l256k", 4000, torch.bfloat16, (262144,) * 8,
                                (1,) * 8, layers=4, **_GLM_DIMS),
    # multi-token (MTP) decode: 32 sequences of 16384 tokens, 4 new query tokens each, drawn
    # independently, and the same with 90% of each token's indexer entries shared with the one
    # before it
    "mtp_b32_l16k_q4": Case("mtp_b32_l16k_q4", 6000, torch.bfloat16, (16384,) * 32, (4,) * 32,
                            **_GLM_DIMS),
    "mtp_b32_l16k_q4_shared": Case("mtp_b32_l16k_q4_shared", 6000, torch.bfloat16,
                                   (16384,) * 32, (4,) * 32, q_share=0.9, **_GLM_DIMS),
    # mixed-length decode, 16 sequences log-uniform in [512, 1048576]
    "mixed_b16_l512_1m": Case("mixed_b16_l512_1m", 5000, torch.bfloat16,
                              tuple(mixed_lengths()), (1,) * 16, **_GLM_DIMS),
}


def custom_case(name: str, seqlens_k, seqlens_q, *, dtype=torch.bfloat16, seed_base=9000,
                layers=1, **dims) -> Case:
    """A case with the decode dims unless overridden (used for edge-case tests)."""
    d = dict(_GLM_DIMS)
    d.update(dims)
    return Case(name, seed_base, dtype, tuple(int(x) for x in seqlens_k),
                tuple(int(x) for x in seqlens_q), layers=layers, **d)


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def uniform_int(shape, lo: int, hi: int, dtype, device, seed: int) -> torch.Tensor:
    """Uniform integers in [lo, hi] cast to ``dtype`` (exact for the small ranges used)."""
    x = torch.randint(lo, hi + 1, tuple(shape), generator=_gen(device, seed), device=device,
                      dtype=torch.int32)
    return x.to(dtype)


def normal(shape, sigma: float, dtype, device, seed: int, chunk_rows: int = 1 << 20) -> torch.Tensor:
    """``randn * sigma`` rounded once to ``dtype``; large tensors are drawn in row chunks from one
    generator so the fp32 temporary stays bounded."""
    shape = tuple(shape)
    g = _gen(device, seed)
    out = torch.empty(shape, dtype=dtype, device=device)
    rows = shape[0]
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        tmp = torch.randn((r1 - r0,) + shape[1:], generator=g, device=device, dtype=torch.float32)
        out[r0:r1] = (tmp * sigma).to(dtype)
    return out


def cu_seqlens(lens, dtype) -> torch.Tensor:
    c = np.zeros(len(lens) + 1, dtype=np.int64)
    c[1:] = np.cumsum(np.asarray(lens, dtype=np.int64))
    return torch.from_numpy(c).to(dtype)


def make_inputs(case: Case, device="cpu", layers: Optional[int] = None) -> Dict[str, object]:
    """All tensors of ``case`` on ``device``.

    Returns a dict with ``q_idx [T,H_I,d_I]``, ``k_idx [total_k,d_I]``, ``w [T,H_I]`` (fp32),
    ``q`` (list over layers of ``[T,H,d_qk]``), ``kv`` (list over layers of ``[total_k,d_qk]``),
    ``cu_seqlens_q`` (int32 [B+1]) and ``cu_seqlens_k`` (int64 [B+1]).
    """
    nl = case.layers if layers is None else layers
    T, K = case.total_q, case.total_k
    sb = case.seed_base
    d = dict(
        q_idx=uniform_int((T, case.index_n_heads, case.index_head_dim), -case.idx_range,
                          case.idx_range, case.dtype, device, sb + ID_Q_IDX),
        k_idx=uniform_int((K, case.index_head_dim), -case.idx_range, case.idx_range, case.dtype,
                          device, sb + ID_K_IDX),
        w=uniform_int((T, case.index_n_heads), -case.w_range, case.w_range, torch.float32, device,
                      sb + ID_W),
        q=[normal((T, case.n_heads, case.d_qk), case.sigma, case.dtype, device, sb + ID_Q0 + l)
           for l in range(nl)],
        kv=[normal((K, case.d_qk), case.sigma, case.dtype, device, sb + ID_KV0 + l)
            for l in range(nl)],
        cu_seqlens_q=cu_seqlens(case.seqlens_q, torch.int32).to(device),
        cu_seqlens_k=cu_seqlens(case.seqlens_k, torch.int64).to(device),
    )
    if case.q_share > 0:
        # correlated query tokens of one sequence (speculative decoding drafts several tokens
        # whose selections overlap): token j > 0 takes each entry of q_I and w from token j-1
        # with probability q_share, element by element, from a generator of its own
        g = _gen(device, sb + ID_SHARE)
        mq = torch.rand(d["q_idx"].shape, generator=g, device=device) < case.q_share
        mw = torch.rand(d["w"].shape, generator=g, device=device) < case.q_share
        t = 0
        for nq in case.seqlens_q:
            for j in range(1, nq):
                d["q_idx"][t + j] = torch.where(mq[t + j], d["q_idx"][t + j - 1], d["q_idx"][t + j])
                d["w"][t + j] = torch.where(mw[t + j], d["w"][t + j - 1], d["w"][t + j])
            t += nq
    return d


def query_rows(case: Case):
    """(t, b, p, key_base) for every query row: query j of sequence b sits at position
    p = L_b - nq_b + j and its key rows start at key_base = cu_seqlens_k[b]."""
    rows = []
    t = 0
    kb = 0
    for b, (L, nq) in enumerate(zip(case.seqlens_k, case.seqlens_q)):
        for j in range(nq):
            rows.append((t, b, L - nq + j, kb))
            t += 1
        kb += L
    return rows

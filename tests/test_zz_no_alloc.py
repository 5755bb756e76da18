"""dsa_sparse_mla_fwd_noalloc (the sparse-MLA call whose split scratch lives in the library's
per-GPU device array instead of a caller workspace) against dsa_sparse_mla_fwd, through the C
ABI, on two calls in a row, the second with a smaller batch: the outputs and log-sum-exps must
be bit-identical (the same kernels run on the same inputs). Named to be collected last."""
import sys
import zlib

import pytest
import torch

import dsa_inputs as DI
import long_context_lightning_amd as dsa

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsa.lib()


def _call_pair(lens, name):
    case = DI.custom_case(name, lens, (1,) * len(lens),
                          seed_base=zlib.crc32(name.encode()) % 100000 * 100)
    say("case", case.name, "lengths", lens)
    d = DI.make_inputs(case, "cuda")
    batch = dsa.Batch(d["cu_seqlens_q"], d["cu_seqlens_k"], 1, max(lens), case.total_q,
                      case.total_k)
    scores = dsa.indexer_scores(d["q_idx"], d["k_idx"], d["w"], batch)
    idx = dsa.topk(scores, batch, case.index_topk)
    T, H = case.total_q, case.n_heads
    need = dsa.workspace_size(dsa.OP_SPARSE_MLA, batch, case.index_topk, H, case.d_v)
    assert 0 < need <= (64 << 20), need          # the call uses the split scratch
    L = dsa.lib()
    sp = torch.cuda.current_stream().cuda_stream
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    ref_o = torch.empty((T, H, case.d_v), dtype=case.dtype, device="cuda")
    ref_l = torch.empty((T, H), dtype=torch.float32, device="cuda")
    st = L.dsa_sparse_mla_fwd(batch.ptr, d["q"][0].data_ptr(), d["kv"][0].data_ptr(),
                              idx.data_ptr(), case.index_topk, H, case.d_qk, case.d_v,
                              case.softmax_scale, 1, ref_o.data_ptr(), ref_l.data_ptr(),
                              ws.data_ptr(), need, sp)
    assert st == 0, st
    out = torch.full((T, H, case.d_v), 7.0, dtype=case.dtype, device="cuda")
    lse = torch.full((T, H), 7.0, dtype=torch.float32, device="cuda")
    st = L.dsa_sparse_mla_fwd_noalloc(batch.ptr, d["q"][0].data_ptr(), d["kv"][0].data_ptr(),
                                      idx.data_ptr(), case.index_topk, H, case.d_qk, case.d_v,
                                      case.softmax_scale, 1, out.data_ptr(), lse.data_ptr(), sp)
    assert st == 0, st
    torch.cuda.synchronize()
    assert torch.equal(out, ref_o), (out.float() - ref_o.float()).abs().max()
    assert torch.equal(lse, ref_l)
    return need


def test_noalloc_matches_workspace_call_twice():
    n1 = _call_pair((9000, 16384, 3000, 12000, 2500, 7000, 16384, 4000) * 2, "noalloc_big")
    n2 = _call_pair((5000, 2100, 9000), "noalloc_small")
    assert n2 < n1
    say("scratch bytes used:", n1, n2)

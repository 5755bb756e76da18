"""C-ABI checks that need no GPU: the library loads, exports every function that
include/dsa.h declares, and rejects invalid arguments on the host with the documented status
before anything is launched (only argument-validation paths are called here)."""
import ctypes
import os
import re

import pytest

import long_context_lightning_amd as dsa
from long_context_lightning_amd import _CBatch, _CForwardArgs

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "dsa.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = 0x1000  # a non-null stand-in; never dereferenced by the validation paths


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(dsa.LIB_PATH):
        pytest.skip("libdsa.so not built")
    return dsa.lib()


def _batch(**kw):
    d = dict(batch=2, total_q=2, total_k=100, max_seqlen_q=1, max_seqlen_k=60,
             cu_seqlens_q=FAKE, cu_seqlens_k=FAKE)
    d.update(kw)
    return _CBatch(d["batch"], d["total_q"], d["total_k"], d["max_seqlen_q"], d["max_seqlen_k"],
                   d["cu_seqlens_q"], d["cu_seqlens_k"])


def test_header_declares_the_path():
    fns = declared_functions()
    for f in ("dsa_indexer_scores", "dsa_topk", "dsa_sparse_mla_fwd", "dsa_forward",
              "dsa_workspace_size", "dsa_check_batch", "dsa_status_string", "dsa_version"):
        assert f in fns


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), f"{name} declared in dsa.h but not exported"


def test_status_strings_and_version(L):
    for code in range(6):
        s = L.dsa_status_string(code).decode()
        assert s.startswith("DSA_")
    assert L.dsa_status_string(99).decode() == "unknown dsa_status"
    assert L.dsa_version() >= 100


def test_indexer_rejects_bad_arguments(L):
    b = _batch()
    f = L.dsa_indexer_scores
    assert f(None, FAKE, FAKE, FAKE, 32, 128, 1, FAKE, 60, None) == INVALID
    assert f(ctypes.byref(b), None, FAKE, FAKE, 32, 128, 1, FAKE, 60, None) == INVALID
    assert f(ctypes.byref(b), FAKE, FAKE, FAKE, 32, 128, 1, None, 60, None) == INVALID
    assert f(ctypes.byref(b), FAKE, FAKE, FAKE, 32, 128, 1, FAKE, 59, None) == INVALID  # ld < L
    assert f(ctypes.byref(b), FAKE, FAKE, FAKE, 48, 128, 1, FAKE, 60, None) == UNSUPPORTED
    assert f(ctypes.byref(b), FAKE, FAKE, FAKE, 32, 64, 1, FAKE, 60, None) == UNSUPPORTED
    assert f(ctypes.byref(b), FAKE, FAKE, FAKE, 32, 128, 7, FAKE, 60, None) == INVALID
    bad = _batch(cu_seqlens_k=None)
    assert f(ctypes.byref(bad), FAKE, FAKE, FAKE, 32, 128, 1, FAKE, 60, None) == INVALID
    bad = _batch(total_q=3, total_k=2)       # more queries than keys
    assert f(ctypes.byref(bad), FAKE, FAKE, FAKE, 32, 128, 1, FAKE, 60, None) == INVALID
    bad = _batch(total_k=121)                # more keys than batch * max_seqlen_k
    assert f(ctypes.byref(bad), FAKE, FAKE, FAKE, 32, 128, 1, FAKE, 60, None) == INVALID


def test_topk_rejects_bad_arguments(L):
    b = _batch()
    f = L.dsa_topk
    assert f(ctypes.byref(b), None, 60, 16, FAKE, None, 0, None) == INVALID
    assert f(ctypes.byref(b), FAKE, 60, 0, FAKE, None, 0, None) == INVALID
    assert f(ctypes.byref(b), FAKE, 60, 16, None, None, 0, None) == INVALID
    assert f(ctypes.byref(b), FAKE, 10, 16, FAKE, None, 0, None) == INVALID


def test_sparse_mla_rejects_bad_arguments(L):
    b = _batch()
    f = L.dsa_sparse_mla_fwd
    args = [ctypes.byref(b), FAKE, FAKE, FAKE, 2048, 64, 576, 512, 1 / 24, 1, FAKE, None, None,
            0, None]
    a = list(args); a[1] = None
    assert f(*a) == INVALID
    a = list(args); a[7] = 600               # d_v > d_qk
    assert f(*a) == INVALID
    a = list(args); a[5] = 48                # heads not a multiple of 32 on bf16
    assert f(*a) == UNSUPPORTED
    a = list(args); a[6] = 512; a[7] = 448   # other latent widths are not compiled
    assert f(*a) == UNSUPPORTED
    for bad in (float("nan"), float("inf"), float("-inf")):   # softmax scale must be finite
        a = list(args); a[8] = bad
        assert f(*a) == INVALID
    a = list(args); a[9] = 0; a[4] = 100000  # fp32 path keeps one softmax row in LDS
    assert f(*a) == UNSUPPORTED
    # 2 decode queries over 64 heads split the selection: a workspace is required
    assert L.dsa_workspace_size(2, ctypes.byref(b), 2048, 64, 512) > 0
    assert f(*args) == WORKSPACE


def test_forward_rejects_bad_arguments(L):
    b = _batch()
    fa = _CForwardArgs(FAKE, FAKE, FAKE, 32, 128, 2048, FAKE, FAKE, 64, 576, 512, 1 / 24, 1)
    f = L.dsa_forward
    assert f(ctypes.byref(b), None, FAKE, 1, FAKE, None, FAKE, 1 << 30, None) == INVALID
    assert f(ctypes.byref(b), ctypes.byref(fa), None, 1, FAKE, None, FAKE, 1 << 30, None) == INVALID
    assert f(ctypes.byref(b), ctypes.byref(fa), FAKE, 2, FAKE, None, FAKE, 1 << 30, None) == INVALID
    assert f(ctypes.byref(b), ctypes.byref(fa), FAKE, 1, FAKE, None, None, 0, None) == WORKSPACE
    fa2 = _CForwardArgs(None, FAKE, FAKE, 32, 128, 2048, FAKE, FAKE, 64, 576, 512, 1 / 24, 1)
    assert f(ctypes.byref(b), ctypes.byref(fa2), FAKE, 1, FAKE, None, FAKE, 1 << 30, None) == INVALID


def test_workspace_sizes(L):
    b = _batch()
    ws = L.dsa_workspace_size
    assert ws(0, ctypes.byref(b), 2048, 64, 512) == 0
    assert ws(0, None, 2048, 64, 512) == 0
    fwd = ws(3, ctypes.byref(b), 2048, 64, 512)
    assert fwd >= 2 * 60 * 4 + ws(2, ctypes.byref(b), 2048, 64, 512)
    assert ws(2, ctypes.byref(b), 2048, 8, 64) == 0      # fp32 path needs no split scratch


def test_sparse_mla_noalloc_rejects_bad_arguments(L):
    """The no-workspace sparse-MLA call validates like the workspace call, on the host, before
    it looks up its device scratch (nothing here reaches a GPU)."""
    b = _batch()
    f = L.dsa_sparse_mla_fwd_noalloc
    args = [ctypes.byref(b), FAKE, FAKE, FAKE, 2048, 64, 576, 512, 1 / 24, 1, FAKE, None, None]
    a = list(args); a[1] = None
    assert f(*a) == INVALID
    a = list(args); a[10] = None                 # no output buffer
    assert f(*a) == INVALID
    a = list(args); a[5] = 48
    assert f(*a) == UNSUPPORTED
    a = list(args); a[8] = float("nan")
    assert f(*a) == INVALID
    assert f(None, *args[1:]) == INVALID


def test_fp8_indexer_rejects_bad_arguments(L):
    b = _batch()
    assert L.dsa_indexer_scores(ctypes.byref(b), FAKE, FAKE, FAKE, 32, 128, 2, FAKE, 60,
                                None) == UNSUPPORTED          # fp8 goes through the _fp8 call
    f = L.dsa_indexer_scores_fp8
    assert f(ctypes.byref(b), None, FAKE, None, FAKE, 32, 128, FAKE, 60, None) == INVALID
    assert f(ctypes.byref(b), FAKE, FAKE, None, None, 32, 128, FAKE, 60, None) == INVALID
    assert f(ctypes.byref(b), FAKE, FAKE, None, FAKE, 32, 128, None, 60, None) == INVALID
    assert f(ctypes.byref(b), FAKE, FAKE, None, FAKE, 32, 128, FAKE, 59, None) == INVALID
    assert f(ctypes.byref(b), FAKE, FAKE, None, FAKE, 48, 128, FAKE, 60, None) == UNSUPPORTED
    assert f(ctypes.byref(b), FAKE, FAKE, None, FAKE, 32, 64, FAKE, 60, None) == UNSUPPORTED
    fa = _CForwardArgs(FAKE, FAKE, FAKE, 32, 128, 2048, FAKE, FAKE, 64, 576, 512, 1 / 24, 1, 2,
                       None)                                   # index_fp8 must be 0 or 1
    assert L.dsa_forward(ctypes.byref(b), ctypes.byref(fa), FAKE, 1, FAKE, None, FAKE, 1 << 30,
                         None) == INVALID


def test_block_topk_rejects_bad_arguments(L):
    b = _batch()
    f = L.dsa_block_topk
    ok = [ctypes.byref(b), FAKE, 60, 64, 0, 32, FAKE, FAKE, 1 << 20, None]
    for i, bad in ((1, None), (6, None), (2, 59), (5, 0), (4, 2)):
        a = list(ok); a[i] = bad
        assert f(*a) == INVALID, i
    for bs in (3, 2, 512, 48):                     # block size: a power of two in 4..256
        a = list(ok); a[3] = bs
        assert f(*a) == UNSUPPORTED, bs
    a = list(ok); a[5] = 1025
    assert f(*a) == UNSUPPORTED
    a = list(ok); a[7] = None
    assert f(*a) == WORKSPACE
    assert L.dsa_block_topk_workspace_size(ctypes.byref(b), 64) == 2 * 1 * 4   # 2 rows x 1 block

"""Python binding of libdsa, the DSA hot path for MI355X (gfx950).

Argument marshalling only: every step runs in the HIP kernels of ``libdsa.so``; torch supplies
device memory and the current stream. The functions mirror the C ABI in ``include/dsa.h``:
``indexer_scores``, ``topk``, ``sparse_mla_fwd`` and ``forward`` (with IndexShare reuse).

Build the library first with ``python -m long_context_lightning_amd.build``; importing works
without it, but every call raises if ``libdsa.so`` is missing.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import torch

__all__ = ["Batch", "indexer_scores", "indexer_scores_fp8", "topk", "block_topk", "sparse_mla_fwd", "sparse_mla_fwd_noalloc",
           "forward", "workspace_size",
           "check_batch", "lib", "LIB_PATH", "DsaError", "OP_INDEXER", "OP_TOPK",
           "OP_SPARSE_MLA", "OP_FORWARD"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdsa.so")

DSA_F32, DSA_BF16, DSA_FP8_E4M3 = 0, 1, 2
FP8_DTYPES = (torch.float8_e4m3fn, torch.uint8)   # OCP e4m3fn bytes
OP_INDEXER, OP_TOPK, OP_SPARSE_MLA, OP_FORWARD = 0, 1, 2, 3

_c = ctypes
_vp = _c.c_void_p


class DsaError(RuntimeError):
    """A libdsa call returned a non-zero status."""

    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {_lib_handle().dsa_status_string(status).decode()}")


class _CBatch(_c.Structure):
    _fields_ = [("batch", _c.c_int32), ("total_q", _c.c_int32), ("total_k", _c.c_int64),
                ("max_seqlen_q", _c.c_int32), ("max_seqlen_k", _c.c_int32),
                ("cu_seqlens_q", _vp), ("cu_seqlens_k", _vp)]


class _CForwardArgs(_c.Structure):
    _fields_ = [("q_idx", _vp), ("k_idx", _vp), ("w", _vp), ("index_n_heads", _c.c_int32),
                ("index_head_dim", _c.c_int32), ("index_topk", _c.c_int32), ("q", _vp),
                ("kv", _vp), ("n_heads", _c.c_int32), ("d_qk", _c.c_int32),
                ("d_v", _c.c_int32), ("softmax_scale", _c.c_float), ("dtype", _c.c_int),
                ("index_fp8", _c.c_int32), ("k_idx_scale", _vp), ("block_size", _c.c_int32),
                ("pool", _c.c_int32)]


_LIB = None


def _lib_handle():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libdsa.so is not built ({LIB_PATH}); run "
                               "`python -m long_context_lightning_amd.build`")
        L = _c.CDLL(LIB_PATH)
        B = _c.POINTER(_CBatch)
        st = _c.c_int
        L.dsa_indexer_scores.argtypes = [B, _vp, _vp, _vp, _c.c_int32, _c.c_int32, _c.c_int, _vp,
                                         _c.c_int64, _vp]
        L.dsa_indexer_scores.restype = st
        L.dsa_indexer_scores_fp8.argtypes = [B, _vp, _vp, _vp, _vp, _c.c_int32, _c.c_int32, _vp,
                                             _c.c_int64, _vp]
        L.dsa_indexer_scores_fp8.restype = st
        L.dsa_topk.argtypes = [B, _vp, _c.c_int64, _c.c_int32, _vp, _vp, _c.c_size_t, _vp]
        L.dsa_topk.restype = st
        L.dsa_block_topk.argtypes = [B, _vp, _c.c_int64, _c.c_int32, _c.c_int, _c.c_int32, _vp,
                                     _vp, _c.c_size_t, _vp]
        L.dsa_block_topk.restype = st
        L.dsa_block_topk_workspace_size.argtypes = [B, _c.c_int32]
        L.dsa_block_topk_workspace_size.restype = _c.c_size_t
        L.dsa_sparse_mla_fwd.argtypes = [B, _vp, _vp, _vp, _c.c_int32, _c.c_int32, _c.c_int32,
                                         _c.c_int32, _c.c_float, _c.c_int, _vp, _vp, _vp,
                                         _c.c_size_t, _vp]
        L.dsa_sparse_mla_fwd.restype = st
        L.dsa_sparse_mla_fwd_noalloc.argtypes = [B, _vp, _vp, _vp, _c.c_int32, _c.c_int32,
                                                 _c.c_int32, _c.c_int32, _c.c_float, _c.c_int,
                                                 _vp, _vp, _vp]
        L.dsa_sparse_mla_fwd_noalloc.restype = st
        L.dsa_forward.argtypes = [B, _c.POINTER(_CForwardArgs), _vp, _c.c_int32, _vp, _vp, _vp,
                                  _c.c_size_t, _vp]
        L.dsa_forward.restype = st
        L.dsa_workspace_size.argtypes = [_c.c_int, B, _c.c_int32, _c.c_int32, _c.c_int32]
        L.dsa_workspace_size.restype = _c.c_size_t
        L.dsa_check_batch.argtypes = [B, _vp]
        L.dsa_check_batch.restype = st
        L.dsa_status_string.argtypes = [_c.c_int]
        L.dsa_status_string.restype = _c.c_char_p
        L.dsa_version.argtypes = []
        L.dsa_version.restype = _c.c_int32
        _LIB = L
    return _LIB


def lib():
    """The loaded ``libdsa.so`` (ctypes.CDLL)."""
    return _lib_handle()


class Batch:
    """Ragged batch: device ``cu_seqlens_q`` (int32 [B+1]) and ``cu_seqlens_k`` (int64 [B+1])
    plus the host sizes the kernels' launch shapes need."""

    def __init__(self, cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor,
                 max_seqlen_q: int, max_seqlen_k: int, total_q: int, total_k: int):
        if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int64:
            raise ValueError("cu_seqlens_q must be int32 and cu_seqlens_k int64")
        if not (cu_seqlens_q.is_cuda and cu_seqlens_k.is_cuda):
            raise ValueError("cu_seqlens must be device tensors")
        self.cu_seqlens_q = cu_seqlens_q.contiguous()
        self.cu_seqlens_k = cu_seqlens_k.contiguous()
        self.batch = cu_seqlens_q.numel() - 1
        self.max_seqlen_q = int(max_seqlen_q)
        self.max_seqlen_k = int(max_seqlen_k)
        self.total_q = int(total_q)
        self.total_k = int(total_k)
        self._c = _CBatch(self.batch, self.total_q, self.total_k, self.max_seqlen_q,
                          self.max_seqlen_k, self.cu_seqlens_q.data_ptr(),
                          self.cu_seqlens_k.data_ptr())

    @classmethod
    def from_lengths(cls, seqlens_q: Sequence[int], seqlens_k: Sequence[int],
                     device="cuda") -> "Batch":
        if len(seqlens_q) != len(seqlens_k) or not len(seqlens_q):
            raise ValueError("seqlens_q and seqlens_k must be non-empty and of equal length")
        cq = [0]
        ck = [0]
        for a, b in zip(seqlens_q, seqlens_k):
            cq.append(cq[-1] + int(a))
            ck.append(ck[-1] + int(b))
        return cls(torch.tensor(cq, dtype=torch.int32, device=device),
                   torch.tensor(ck, dtype=torch.int64, device=device),
                   max(seqlens_q), max(seqlens_k), cq[-1], ck[-1])

    @property
    def ptr(self):
        return _c.byref(self._c)


def _stream(t: torch.Tensor):
    return _vp(torch.cuda.current_stream(t.device).cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DSA_BF16
    if t.dtype == torch.float32:
        return DSA_F32
    raise ValueError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _need(t: torch.Tensor, name: str, shape=None, dtype=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None:
        if t.dim() != len(shape) or any(s is not None and s != d for s, d in zip(shape, t.shape)):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")


def _check(status: int, what: str):
    if status != 0:
        raise DsaError(status, what)


def workspace_size(op: int, batch: Batch, index_topk: int, n_heads: int = 0, d_v: int = 0) -> int:
    return int(_lib_handle().dsa_workspace_size(op, batch.ptr, index_topk, n_heads, d_v))


def _workspace(nbytes: int, device) -> Tuple[Optional[torch.Tensor], int]:
    if nbytes <= 0:
        return None, 0
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


def indexer_scores(q_idx: torch.Tensor, k_idx: torch.Tensor, w: torch.Tensor, batch: Batch,
                   ld: Optional[int] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Lightning-indexer scores [T, ld] fp32; entry (t, s) is written for s <= p(t) only."""
    T = batch.total_q
    _need(q_idx, "q_idx", (T, None, None))
    H_I, d_I = q_idx.shape[1], q_idx.shape[2]
    _need(k_idx, "k_idx", (batch.total_k, d_I), q_idx.dtype)
    _need(w, "w", (T, H_I), torch.float32)
    ld = batch.max_seqlen_k if ld is None else int(ld)
    if out is None:
        out = torch.empty((T, ld), dtype=torch.float32, device=q_idx.device)
    _need(out, "scores", (T, ld), torch.float32)
    _check(_lib_handle().dsa_indexer_scores(batch.ptr, q_idx.data_ptr(), k_idx.data_ptr(),
                                            w.data_ptr(), H_I, d_I, _dtype_code(q_idx),
                                            out.data_ptr(), ld, _stream(q_idx)),
           "dsa_indexer_scores")
    return out


def indexer_scores_fp8(q_idx: torch.Tensor, k_idx: torch.Tensor, w: torch.Tensor, batch: Batch,
                       k_scale: Optional[torch.Tensor] = None, ld: Optional[int] = None,
                       out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Lightning-indexer scores from fp8 e4m3fn ``q_idx`` / ``k_idx`` (torch.float8_e4m3fn or
    their uint8 bytes) with optional per-key scales ``k_scale`` [total_k] fp32."""
    T = batch.total_q
    _need(q_idx, "q_idx", (T, None, None))
    if q_idx.dtype not in FP8_DTYPES or k_idx.dtype not in FP8_DTYPES:
        raise ValueError("q_idx and k_idx must be float8_e4m3fn (or their uint8 bytes)")
    H_I, d_I = q_idx.shape[1], q_idx.shape[2]
    _need(k_idx, "k_idx", (batch.total_k, d_I))
    _need(w, "w", (T, H_I), torch.float32)
    if k_scale is not None:
        _need(k_scale, "k_scale", (batch.total_k,), torch.float32)
    ld = batch.max_seqlen_k if ld is None else int(ld)
    if out is None:
        out = torch.empty((T, ld), dtype=torch.float32, device=q_idx.device)
    _need(out, "scores", (T, ld), torch.float32)
    _check(_lib_handle().dsa_indexer_scores_fp8(
        batch.ptr, q_idx.data_ptr(), k_idx.data_ptr(),
        k_scale.data_ptr() if k_scale is not None else None, w.data_ptr(), H_I, d_I,
        out.data_ptr(), ld, _stream(q_idx)), "dsa_indexer_scores_fp8")
    return out


def topk(scores: torch.Tensor, batch: Batch, index_topk: int,
         out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Causal top-k indices [T, index_topk] int32 (ascending, -1 padded)."""
    T = batch.total_q
    _need(scores, "scores", (T, None), torch.float32)
    if out is None:
        out = torch.empty((T, index_topk), dtype=torch.int32, device=scores.device)
    _need(out, "indices", (T, index_topk), torch.int32)
    ws, nb = _workspace(workspace_size(OP_TOPK, batch, index_topk), scores.device)
    _check(_lib_handle().dsa_topk(batch.ptr, scores.data_ptr(), scores.shape[1], index_topk,
                                  out.data_ptr(), ws.data_ptr() if ws is not None else None, nb,
                                  _stream(scores)), "dsa_topk")
    return out


POOL_MAX, POOL_MEAN = 0, 1


def block_topk(scores: torch.Tensor, batch: Batch, block_size: int, topk_blocks: int,
               pool: str = "max", out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Block-pooled selection: every visible position of the ``topk_blocks`` best blocks of
    ``block_size`` positions (block score = max or mean of its scores), [T, topk_blocks *
    block_size] int32, ascending, -1 padded."""
    T = batch.total_q
    _need(scores, "scores", (T, None), torch.float32)
    if pool not in ("max", "mean"):
        raise ValueError("pool must be 'max' or 'mean'")
    n = topk_blocks * block_size
    if out is None:
        out = torch.empty((T, n), dtype=torch.int32, device=scores.device)
    _need(out, "indices", (T, n), torch.int32)
    L = _lib_handle()
    nb = int(L.dsa_block_topk_workspace_size(batch.ptr, block_size))
    ws, nb = _workspace(nb, scores.device)
    _check(L.dsa_block_topk(batch.ptr, scores.data_ptr(), scores.shape[1], block_size,
                            POOL_MEAN if pool == "mean" else POOL_MAX, topk_blocks,
                            out.data_ptr(), ws.data_ptr() if ws is not None else None, nb,
                            _stream(scores)), "dsa_block_topk")
    return out


def sparse_mla_fwd(q: torch.Tensor, kv: torch.Tensor, indices: torch.Tensor, batch: Batch,
                   softmax_scale: float, d_v: int, out: Optional[torch.Tensor] = None,
                   return_lse: bool = True):
    """Sparse MQA attention over the selected latent rows: (out [T,H,d_v], lse [T,H] or None)."""
    T = batch.total_q
    _need(q, "q", (T, None, None))
    H, d_qk = q.shape[1], q.shape[2]
    _need(kv, "kv", (batch.total_k, d_qk), q.dtype)
    _need(indices, "indices", (T, None), torch.int32)
    k = indices.shape[1]
    if out is None:
        out = torch.empty((T, H, d_v), dtype=q.dtype, device=q.device)
    _need(out, "out", (T, H, d_v), q.dtype)
    lse = torch.empty((T, H), dtype=torch.float32, device=q.device) if return_lse else None
    ws, nb = _workspace(workspace_size(OP_SPARSE_MLA, batch, k, H, d_v), q.device)
    _check(_lib_handle().dsa_sparse_mla_fwd(
        batch.ptr, q.data_ptr(), kv.data_ptr(), indices.data_ptr(), k, H, d_qk, d_v,
        float(softmax_scale), _dtype_code(q), out.data_ptr(),
        lse.data_ptr() if lse is not None else None,
        ws.data_ptr() if ws is not None else None, nb, _stream(q)), "dsa_sparse_mla_fwd")
    return out, lse


def sparse_mla_fwd_noalloc(q: torch.Tensor, kv: torch.Tensor, indices: torch.Tensor,
                           batch: Batch, softmax_scale: float, d_v: int, out: torch.Tensor,
                           lse: Optional[torch.Tensor] = None):
    """``sparse_mla_fwd`` into caller-provided ``out`` (and ``lse``) with the library's own
    per-GPU scratch: no workspace is passed and nothing is allocated."""
    T = batch.total_q
    _need(q, "q", (T, None, None))
    H, d_qk = q.shape[1], q.shape[2]
    _need(kv, "kv", (batch.total_k, d_qk), q.dtype)
    _need(indices, "indices", (T, None), torch.int32)
    _need(out, "out", (T, H, d_v), q.dtype)
    if lse is not None:
        _need(lse, "lse", (T, H), torch.float32)
    _check(_lib_handle().dsa_sparse_mla_fwd_noalloc(
        batch.ptr, q.data_ptr(), kv.data_ptr(), indices.data_ptr(), indices.shape[1], H, d_qk,
        d_v, float(softmax_scale), _dtype_code(q), out.data_ptr(),
        lse.data_ptr() if lse is not None else None, _stream(q)), "dsa_sparse_mla_fwd_noalloc")
    return out, lse


def forward(q: torch.Tensor, kv: torch.Tensor, batch: Batch, index_topk: int,
            softmax_scale: float, d_v: int, *, q_idx: Optional[torch.Tensor] = None,
            k_idx: Optional[torch.Tensor] = None, w: Optional[torch.Tensor] = None,
            shared_indices: Optional[torch.Tensor] = None, compute_indices: bool = True,
            out: Optional[torch.Tensor] = None, return_lse: bool = True,
            workspace: Optional[torch.Tensor] = None, k_idx_scale: Optional[torch.Tensor] = None,
            block_size: int = 0, pool: str = "max"):
    """Indexer -> top-k -> sparse MLA in one call.

    With ``compute_indices`` the indexer and top-k fill ``shared_indices`` (allocated if None);
    without it the cached ``shared_indices`` of an earlier layer of the IndexShare group are
    reused. fp8 (float8_e4m3fn) ``q_idx`` / ``k_idx`` select the fp8 indexer, with optional
    per-key scales ``k_idx_scale``. ``block_size`` > 0 selects whole blocks (dsa_block_topk:
    index_topk / block_size blocks, ``pool`` 'max' or 'mean'). Returns (out, lse,
    shared_indices).
    """
    T = batch.total_q
    _need(q, "q", (T, None, None))
    H, d_qk = q.shape[1], q.shape[2]
    _need(kv, "kv", (batch.total_k, d_qk), q.dtype)
    if shared_indices is None:
        if not compute_indices:
            raise ValueError("compute_indices=False needs the cached shared_indices")
        shared_indices = torch.empty((T, index_topk), dtype=torch.int32, device=q.device)
    _need(shared_indices, "shared_indices", (T, index_topk), torch.int32)
    H_I = d_I = 0
    fp8 = False
    if compute_indices:
        fp8 = q_idx is not None and q_idx.dtype in FP8_DTYPES
        _need(q_idx, "q_idx", (T, None, None), None if fp8 else q.dtype)
        H_I, d_I = q_idx.shape[1], q_idx.shape[2]
        _need(k_idx, "k_idx", (batch.total_k, d_I), None if fp8 else q.dtype)
        if fp8 and k_idx.dtype not in FP8_DTYPES:
            raise ValueError("q_idx and k_idx must both be fp8")
        _need(w, "w", (T, H_I), torch.float32)
        if k_idx_scale is not None:
            if not fp8:
                raise ValueError("k_idx_scale applies to fp8 indexer inputs only")
            _need(k_idx_scale, "k_idx_scale", (batch.total_k,), torch.float32)
    if out is None:
        out = torch.empty((T, H, d_v), dtype=q.dtype, device=q.device)
    _need(out, "out", (T, H, d_v), q.dtype)
    lse = torch.empty((T, H), dtype=torch.float32, device=q.device) if return_lse else None
    need = workspace_size(OP_FORWARD, batch, index_topk, H, d_v)
    if workspace is None:
        workspace, nb = _workspace(need, q.device)
    else:
        _need(workspace, "workspace", None, torch.uint8)
        nb = workspace.numel()
    args = _CForwardArgs(
        q_idx.data_ptr() if compute_indices else None, k_idx.data_ptr() if compute_indices else None,
        w.data_ptr() if compute_indices else None, H_I, d_I, index_topk, q.data_ptr(),
        kv.data_ptr(), H, d_qk, d_v, float(softmax_scale), _dtype_code(q), 1 if fp8 else 0,
        k_idx_scale.data_ptr() if (fp8 and k_idx_scale is not None) else None, int(block_size),
        POOL_MEAN if pool == "mean" else POOL_MAX)
    _check(_lib_handle().dsa_forward(batch.ptr, _c.byref(args), shared_indices.data_ptr(),
                                     1 if compute_indices else 0, out.data_ptr(),
                                     lse.data_ptr() if lse is not None else None,
                                     workspace.data_ptr() if workspace is not None else None, nb,
                                     _stream(q)), "dsa_forward")
    return out, lse, shared_indices


def check_batch(batch: Batch) -> None:
    """Validate cu_seqlens against the host sizes (synchronises the current stream)."""
    _check(_lib_handle().dsa_check_batch(batch.ptr, _stream(batch.cu_seqlens_q)),
           "dsa_check_batch")

"""MiniMax Sparse Attention (MSA) forward path on AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libmsa.so``: the functions below carry the names
of the C entry points declared in ``include/msa.h`` and only marshal
arguments.  Every step of the computation runs in the library's HIP kernels;
torch is used for device memory and the current stream.  There is no fallback:
if the library is missing, importing its functions raises.
"""
from __future__ import annotations

import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmsa.so")

MSA_OK = 0
STATUS_NAMES = {0: "MSA_OK", 1: "MSA_ERR_NULL_PTR", 2: "MSA_ERR_INVALID_DIMS", 3: "MSA_ERR_UNSUPPORTED",
                4: "MSA_ERR_MISALIGNED", 5: "MSA_ERR_WORKSPACE_TOO_SMALL", 6: "MSA_ERR_HIP"}
ENTRY_INDEX_SCORES, ENTRY_BLOCK_TOPK, ENTRY_SPARSE_ATTN_FWD, ENTRY_FORWARD, ENTRY_KL_LOSS_FWD = 0, 1, 2, 3, 4
ENTRY_SPARSE_ATTN_BWD, ENTRY_KL_LOSS_BWD = 5, 6
EXPORTED = ("msa_index_scores", "msa_block_topk", "msa_sparse_attn_fwd", "msa_forward",
            "msa_forward_profiled", "msa_attn_chunks", "msa_workspace_bytes", "msa_status_str",
            "msa_block_mask", "msa_mask_blocks", "msa_kl_loss_fwd", "msa_sparse_attn_bwd",
            "msa_kl_loss_bwd")
STAGES = ("index_scores", "block_topk", "attn_build", "attn_partial", "attn_merge")


class MsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}")


class Dims(ctypes.Structure):
    """``msa_dims`` of include/msa.h."""
    _fields_ = [("batch", ctypes.c_int32), ("seqlen_q", ctypes.c_int32), ("seqlen_k", ctypes.c_int32),
                ("num_heads_q", ctypes.c_int32), ("num_heads_kv", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("index_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("topk", ctypes.c_int32), ("causal", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float)]

    @classmethod
    def make(cls, batch, seqlen_q, seqlen_k, num_heads_q, num_heads_kv, head_dim=128, index_dim=128,
             block_size=128, topk=16, causal=1, softmax_scale=0.0):
        return cls(batch, seqlen_q, seqlen_k, num_heads_q, num_heads_kv, head_dim, index_dim,
                   block_size, topk, causal, softmax_scale)

    @property
    def n_blk(self):
        return -(-self.seqlen_k // self.block_size)


_lib = None


def lib():
    """The loaded ``libmsa.so`` (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, D = ctypes.c_void_p, ctypes.POINTER(Dims)
        L.msa_index_scores.argtypes = [D, P, P, P, P]
        L.msa_block_topk.argtypes = [D, P, P, P]
        L.msa_sparse_attn_fwd.argtypes = [D, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.msa_forward.argtypes = [D, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.msa_forward_profiled.argtypes = [D, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P,
                                           ctypes.POINTER(ctypes.c_void_p), ctypes.c_int]
        L.msa_block_mask.argtypes = [D, P, P, P]
        L.msa_mask_blocks.argtypes = [D, P, P, P]
        L.msa_kl_loss_fwd.argtypes = [D, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.msa_kl_loss_bwd.argtypes = [D, P, P, P, P, P, P, P, ctypes.c_float, P, P, P, ctypes.c_size_t, P]
        L.msa_sparse_attn_bwd.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        for f in (L.msa_index_scores, L.msa_block_topk, L.msa_sparse_attn_fwd, L.msa_forward,
                  L.msa_forward_profiled, L.msa_block_mask, L.msa_mask_blocks, L.msa_kl_loss_fwd,
                  L.msa_sparse_attn_bwd, L.msa_kl_loss_bwd):
            f.restype = ctypes.c_int
        L.msa_attn_chunks.argtypes = [D]
        L.msa_attn_chunks.restype = ctypes.c_int
        L.msa_workspace_bytes.argtypes = [D, ctypes.c_int]
        L.msa_workspace_bytes.restype = ctypes.c_size_t
        L.msa_status_str.argtypes = [ctypes.c_int]
        L.msa_status_str.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _check(rc, where):
    if rc != MSA_OK:
        raise MsaError(rc, where)


def _bf16_cuda(name, t, ndim):
    import torch
    if not (t.is_cuda and t.dtype == torch.bfloat16 and t.is_contiguous() and t.dim() == ndim):
        raise ValueError(f"{name} must be a contiguous {ndim}-d bf16 CUDA tensor")


def msa_status_str(status: int) -> str:
    return lib().msa_status_str(status).decode()


def msa_workspace_bytes(dims: Dims, entry: int) -> int:
    n = lib().msa_workspace_bytes(ctypes.byref(dims), entry)
    if n == (1 << 64) - 1:
        raise MsaError(2, "msa_workspace_bytes")
    return n


def dims_of(q=None, k=None, q_idx=None, k_idx=None, *, topk=16, block_size=128, softmax_scale=0.0):
    """msa_dims from tensors laid out as include/msa.h states."""
    if q is not None:
        B, Sq, Hq, D = q.shape
        Sk, Hkv = k.shape[1], k.shape[2]
    else:
        B, Sq, Hkv, _ = q_idx.shape
        Sk, Hq, D = k_idx.shape[1], Hkv, 128
    Didx = q_idx.shape[-1] if q_idx is not None else 128
    return Dims.make(B, Sq, Sk, Hq, Hkv, D, Didx, block_size, topk, 1, softmax_scale)


def _workspace(dims, entry, ws, dev):
    import torch
    need = msa_workspace_bytes(dims, entry)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    return ws, ws.numel() * ws.element_size()


def msa_index_scores(q_idx, k_idx, *, block_size=128, topk=16, block_scores=None):
    """Block scores [B, H_kv, S_q, n_blk] fp32 of the index branch."""
    import torch
    _bf16_cuda("q_idx", q_idx, 4)
    _bf16_cuda("k_idx", k_idx, 3)
    d = dims_of(q_idx=q_idx, k_idx=k_idx, topk=topk, block_size=block_size)
    shape = (d.batch, d.num_heads_kv, d.seqlen_q, d.n_blk)
    if block_scores is None:
        block_scores = torch.empty(shape, dtype=torch.float32, device=q_idx.device)
    rc = lib().msa_index_scores(ctypes.byref(d), _ptr(q_idx), _ptr(k_idx), _ptr(block_scores),
                                _stream(q_idx.device))
    _check(rc, "msa_index_scores")
    return block_scores


def msa_block_topk(block_scores, *, seqlen_k, topk=16, block_size=128, block_idx=None):
    """Selected blocks [B, H_kv, S_q, topk] int32 (ascending, -1 padded)."""
    import torch
    B, Hkv, Sq, nb = block_scores.shape
    d = Dims.make(B, Sq, seqlen_k, Hkv, Hkv, 128, 128, block_size, topk, 1, 0.0)
    if nb != d.n_blk:
        raise ValueError("block_scores last dim must be ceil(seqlen_k / block_size)")
    if block_idx is None:
        block_idx = torch.empty((B, Hkv, Sq, topk), dtype=torch.int32, device=block_scores.device)
    rc = lib().msa_block_topk(ctypes.byref(d), _ptr(block_scores), _ptr(block_idx),
                              _stream(block_scores.device))
    _check(rc, "msa_block_topk")
    return block_idx


def _selection_dims(B, Hkv, Sq, seqlen_k, topk, block_size):
    return Dims.make(B, Sq, seqlen_k, Hkv, Hkv, 128, 128, block_size, topk, 1, 0.0)


def msa_block_mask(block_idx, *, seqlen_k, block_size=128, mask=None):
    """Block-mask form [B, H_kv, S_q, ceil(n_blk / 32)] (int32 tensor holding
    uint32 words) of a selection [B, H_kv, S_q, topk]."""
    import torch
    B, Hkv, Sq, topk = block_idx.shape
    d = _selection_dims(B, Hkv, Sq, seqlen_k, topk, block_size)
    if mask is None:
        mask = torch.empty((B, Hkv, Sq, -(-d.n_blk // 32)), dtype=torch.int32, device=block_idx.device)
    rc = lib().msa_block_mask(ctypes.byref(d), _ptr(block_idx), _ptr(mask), _stream(block_idx.device))
    _check(rc, "msa_block_mask")
    return mask


def msa_mask_blocks(mask, *, seqlen_k, topk=16, block_size=128, block_idx=None):
    """Traversal of block masks [B, H_kv, S_q, n_words]: the set blocks in
    ascending order, at most topk per row, -1 padded -> [B, H_kv, S_q, topk]."""
    import torch
    B, Hkv, Sq, nw = mask.shape
    d = _selection_dims(B, Hkv, Sq, seqlen_k, topk, block_size)
    if nw != -(-d.n_blk // 32):
        raise ValueError("mask last dim must be ceil(ceil(seqlen_k / block_size) / 32)")
    if block_idx is None:
        block_idx = torch.empty((B, Hkv, Sq, topk), dtype=torch.int32, device=mask.device)
    rc = lib().msa_mask_blocks(ctypes.byref(d), _ptr(mask), _ptr(block_idx), _stream(mask.device))
    _check(rc, "msa_mask_blocks")
    return block_idx


def msa_sparse_attn_fwd(q, k, v, block_idx, *, block_size=128, softmax_scale=0.0, out=None,
                        return_lse=False, workspace=None):
    """Main-branch attention over the selected blocks; returns out (and lse)."""
    import torch
    for n, t in (("q", q), ("k", k), ("v", v)):
        _bf16_cuda(n, t, 4)
    d = dims_of(q, k, topk=block_idx.shape[-1], block_size=block_size, softmax_scale=softmax_scale)
    d.index_dim = 128
    if out is None:
        out = torch.empty_like(q)
    lse = torch.empty((d.batch, d.num_heads_q, d.seqlen_q), dtype=torch.float32, device=q.device) \
        if return_lse else None
    ws, nbytes = _workspace(d, ENTRY_SPARSE_ATTN_FWD, workspace, q.device)
    rc = lib().msa_sparse_attn_fwd(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(block_idx),
                                   _ptr(out), _ptr(lse), _ptr(ws), nbytes, _stream(q.device))
    _check(rc, "msa_sparse_attn_fwd")
    return (out, lse) if return_lse else out


def msa_attn_chunks(dims: Dims) -> int:
    """Query chunks the attention stages run in for these dims."""
    return lib().msa_attn_chunks(ctypes.byref(dims))


def msa_forward(q, k, v, q_idx, k_idx, *, topk=16, block_size=128, softmax_scale=0.0, out=None,
                return_lse=False, return_idx=False, workspace=None, stage_events=None):
    """Index scores -> Top-k -> sparse attention.  Returns out, plus lse and
    block_idx when asked."""
    import torch
    for n, t, nd in (("q", q, 4), ("k", k, 4), ("v", v, 4), ("q_idx", q_idx, 4), ("k_idx", k_idx, 3)):
        _bf16_cuda(n, t, nd)
    d = dims_of(q, k, q_idx, k_idx, topk=topk, block_size=block_size, softmax_scale=softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    lse = torch.empty((d.batch, d.num_heads_q, d.seqlen_q), dtype=torch.float32, device=q.device) \
        if return_lse else None
    idx = torch.empty((d.batch, d.num_heads_kv, d.seqlen_q, topk), dtype=torch.int32, device=q.device) \
        if return_idx else None
    ws, nbytes = _workspace(d, ENTRY_FORWARD, workspace, q.device)
    args = (ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(q_idx), _ptr(k_idx), _ptr(out), _ptr(lse),
            _ptr(idx), _ptr(ws), nbytes, _stream(q.device))
    if stage_events is None:
        rc = lib().msa_forward(*args)
        _check(rc, "msa_forward")
    else:
        # stage_events: 2 * len(STAGES) raw hipEvent_t handles (msa_forward_profiled).
        arr = (ctypes.c_void_p * len(stage_events))(*stage_events)
        rc = lib().msa_forward_profiled(*args, arr, len(stage_events))
        _check(rc, "msa_forward_profiled")
    res = [out]
    if return_lse:
        res.append(lse)
    if return_idx:
        res.append(idx)
    return res[0] if len(res) == 1 else tuple(res)


def default_softmax_scale(head_dim: int = 128) -> float:
    return 1.0 / math.sqrt(head_dim)


def msa_kl_loss_fwd(q, k, q_idx, k_idx, block_idx, lse, *, block_size=128, softmax_scale=0.0,
                    return_rows=False, return_lse_idx=False, workspace=None):
    """Alignment loss of the index branch (forward value): the mean over
    (batch, query, group) rows of KL(group-mean main-branch probabilities ||
    softmax of the index scores) on each row's selected tokens.  ``lse`` is
    the main branch's log-sum-exp over the same selection ([B, H_q, S_q], as
    msa_forward returns it).  Returns the loss as a 0-d fp32 tensor, then the
    per-row terms [B, H_kv, S_q] when return_rows is set and the rows'
    log-sum-exps of the index scores [B, H_kv, S_q] when return_lse_idx is."""
    import torch
    for n, t, nd in (("q", q, 4), ("k", k, 4), ("q_idx", q_idx, 4), ("k_idx", k_idx, 3)):
        _bf16_cuda(n, t, nd)
    d = dims_of(q, k, q_idx, k_idx, topk=block_idx.shape[-1], block_size=block_size,
                softmax_scale=softmax_scale)
    for n, t, dt in (("block_idx", block_idx, torch.int32), ("lse", lse, torch.float32)):
        if not (t.is_cuda and t.dtype == dt and t.is_contiguous()):
            raise ValueError(f"{n} must be a contiguous {dt} CUDA tensor")
    if tuple(lse.shape) != (d.batch, d.num_heads_q, d.seqlen_q):
        raise ValueError("lse must be [B, H_q, S_q]")
    if tuple(block_idx.shape[:3]) != (d.batch, d.num_heads_kv, d.seqlen_q):
        raise ValueError("block_idx must be [B, H_kv, S_q, topk]")
    loss = torch.empty((), dtype=torch.float32, device=q.device)
    shape = (d.batch, d.num_heads_kv, d.seqlen_q)
    rows = torch.empty(shape, dtype=torch.float32, device=q.device) if return_rows else None
    lse_idx = torch.empty(shape, dtype=torch.float32, device=q.device) if return_lse_idx else None
    ws, nbytes = _workspace(d, ENTRY_KL_LOSS_FWD, workspace, q.device)
    rc = lib().msa_kl_loss_fwd(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(q_idx), _ptr(k_idx),
                               _ptr(block_idx), _ptr(lse), _ptr(rows), _ptr(loss), _ptr(lse_idx), _ptr(ws),
                               nbytes, _stream(q.device))
    _check(rc, "msa_kl_loss_fwd")
    res = [loss] + ([rows] if return_rows else []) + ([lse_idx] if return_lse_idx else [])
    return res[0] if len(res) == 1 else tuple(res)


def msa_sparse_attn_bwd(q, k, v, block_idx, out, lse, dout, *, block_size=128, softmax_scale=0.0,
                        workspace=None):
    """Main-branch backward over the selection: returns (dq, dk, dv), bf16,
    from the upstream gradient dout and the forward's out and lse."""
    import torch
    for n, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
        _bf16_cuda(n, t, 4)
    d = dims_of(q, k, topk=block_idx.shape[-1], block_size=block_size, softmax_scale=softmax_scale)
    d.index_dim = 128
    for n, t, dt in (("block_idx", block_idx, torch.int32), ("lse", lse, torch.float32)):
        if not (t.is_cuda and t.dtype == dt and t.is_contiguous()):
            raise ValueError(f"{n} must be a contiguous {dt} CUDA tensor")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws, nbytes = _workspace(d, ENTRY_SPARSE_ATTN_BWD, workspace, q.device)
    rc = lib().msa_sparse_attn_bwd(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(block_idx), _ptr(out),
                                   _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), nbytes,
                                   _stream(q.device))
    _check(rc, "msa_sparse_attn_bwd")
    return dq, dk, dv


def msa_kl_loss_bwd(q, k, q_idx, k_idx, block_idx, lse, lse_idx, grad_loss=1.0, *, block_size=128,
                    softmax_scale=0.0, workspace=None):
    """Gradient of grad_loss * (the alignment loss) with respect to q_idx and
    k_idx, the teacher detached: returns (dq_idx, dk_idx), bf16.  lse is the
    main branch's LSE and lse_idx the index scores' LSE of msa_kl_loss_fwd."""
    import torch
    for n, t, nd in (("q", q, 4), ("k", k, 4), ("q_idx", q_idx, 4), ("k_idx", k_idx, 3)):
        _bf16_cuda(n, t, nd)
    d = dims_of(q, k, q_idx, k_idx, topk=block_idx.shape[-1], block_size=block_size,
                softmax_scale=softmax_scale)
    for n, t, dt in (("block_idx", block_idx, torch.int32), ("lse", lse, torch.float32),
                     ("lse_idx", lse_idx, torch.float32)):
        if not (t.is_cuda and t.dtype == dt and t.is_contiguous()):
            raise ValueError(f"{n} must be a contiguous {dt} CUDA tensor")
    dq_idx, dk_idx = torch.empty_like(q_idx), torch.empty_like(k_idx)
    ws, nbytes = _workspace(d, ENTRY_KL_LOSS_BWD, workspace, q.device)
    rc = lib().msa_kl_loss_bwd(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(q_idx), _ptr(k_idx), _ptr(block_idx),
                               _ptr(lse), _ptr(lse_idx), float(grad_loss), _ptr(dq_idx), _ptr(dk_idx), _ptr(ws),
                               nbytes, _stream(q.device))
    _check(rc, "msa_kl_loss_bwd")
    return dq_idx, dk_idx

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
ENTRY_SPARSE_ATTN_BWD, ENTRY_KL_LOSS_BWD, ENTRY_BACKWARD = 5, 6, 7
EXPORTED = ("msa_index_scores", "msa_block_topk", "msa_sparse_attn_fwd", "msa_forward",
            "msa_forward_profiled", "msa_attn_chunks", "msa_workspace_bytes", "msa_workspace_min_bytes",
            "msa_status_str", "msa_block_mask", "msa_mask_blocks", "msa_kl_loss_fwd", "msa_sparse_attn_bwd",
            "msa_kl_loss_bwd", "msa_forward_noalloc", "msa_backward")
NOALLOC_SCRATCH_BYTES = 256 << 20  # MSA_NOALLOC_SCRATCH_BYTES of msa.h
# Stages of msa_forward_profiled: the index scores and the Top-k once, then the
# three attention stages once per query chunk.
STAGES = ("index_scores", "block_topk", "attn_build", "attn_partial", "attn_merge")
ATTN_STAGES = STAGES[2:]


def n_stage_events(chunks: int) -> int:
    """Events msa_forward_profiled records for a forward in `chunks` query chunks."""
    return 4 + 6 * chunks


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
        L.msa_forward_noalloc.argtypes = [D, P, P, P, P, P, P, P, P, P]
        L.msa_block_mask.argtypes = [D, P, P, P]
        L.msa_mask_blocks.argtypes = [D, P, P, P]
        L.msa_kl_loss_fwd.argtypes = [D, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.msa_kl_loss_bwd.argtypes = [D, P, P, P, P, P, P, P, ctypes.c_float, P, P, P, ctypes.c_size_t, P]
        L.msa_sparse_attn_bwd.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.msa_backward.argtypes = [D, P, P, P, P, P, P, P, P, P, P, ctypes.c_float, P, P, P, P, P, P,
                                   ctypes.c_size_t, P]
        for f in (L.msa_index_scores, L.msa_block_topk, L.msa_sparse_attn_fwd, L.msa_forward,
                  L.msa_forward_profiled, L.msa_block_mask, L.msa_mask_blocks, L.msa_kl_loss_fwd,
                  L.msa_sparse_attn_bwd, L.msa_kl_loss_bwd, L.msa_forward_noalloc, L.msa_backward):
            f.restype = ctypes.c_int
        L.msa_attn_chunks.argtypes = [D, ctypes.c_int, ctypes.c_size_t]
        L.msa_attn_chunks.restype = ctypes.c_int
        for f in (L.msa_workspace_bytes, L.msa_workspace_min_bytes):
            f.argtypes = [D, ctypes.c_int]
            f.restype = ctypes.c_size_t
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




# ------------------------------------------------------------ validation
# Every tensor argument is checked against the shape msa.h gives it before the
# library sees its pointer: dtype first, then the exact shape, contiguity and
# the device (so a mistake is reported the same way on a host without a GPU).
def _expect(name, t, dtype, shape, device=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the other arguments on {device}")


def _rank(name, t, ndim):
    import torch
    if not isinstance(t, torch.Tensor) or t.dim() != ndim:
        raise ValueError(f"{name} must be a {ndim}-d tensor")


def _out(name, t, dtype, shape, device):
    """A caller-provided output (checked like an input) or a new one."""
    import torch
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _expect(name, t, dtype, shape, device)
    return t


def msa_status_str(status: int) -> str:
    return lib().msa_status_str(status).decode()


def msa_workspace_bytes(dims: Dims, entry: int) -> int:
    """Workspace size the entry point is designed for (msa.h)."""
    n = lib().msa_workspace_bytes(ctypes.byref(dims), entry)
    if n == (1 << 64) - 1:
        raise MsaError(2, "msa_workspace_bytes")
    return n


def msa_workspace_min_bytes(dims: Dims, entry: int) -> int:
    """The smallest workspace the entry point accepts (msa.h)."""
    n = lib().msa_workspace_min_bytes(ctypes.byref(dims), entry)
    if n == (1 << 64) - 1:
        raise MsaError(2, "msa_workspace_min_bytes")
    return n


def msa_attn_chunks(dims: Dims, entry: int = ENTRY_FORWARD, ws_bytes: int | None = None) -> int:
    """Query chunks the entry point runs in with ws_bytes of workspace (the
    designed size when None); 0 when the dims or the size are not valid."""
    if ws_bytes is None:
        n = lib().msa_workspace_bytes(ctypes.byref(dims), entry)
        if n == (1 << 64) - 1:
            return 0
        ws_bytes = n
    return lib().msa_attn_chunks(ctypes.byref(dims), entry, ws_bytes)


def dims_of(q=None, k=None, q_idx=None, k_idx=None, *, topk=16, block_size=128, softmax_scale=0.0):
    """msa_dims from tensors laid out as include/msa.h states (shapes only)."""
    if q is not None:
        _rank("q", q, 4)
        _rank("k", k, 4)
        B, Sq, Hq, D = q.shape
        Sk, Hkv = k.shape[1], k.shape[2]
    else:
        _rank("q_idx", q_idx, 4)
        _rank("k_idx", k_idx, 3)
        B, Sq, Hkv, _ = q_idx.shape
        Sk, Hq, D = k_idx.shape[1], Hkv, 128
    Didx = q_idx.shape[-1] if q_idx is not None else 128
    return Dims.make(B, Sq, Sk, Hq, Hkv, D, Didx, block_size, topk, 1, softmax_scale)


def _main_inputs(d, dev, **ts):
    """Checks the main-branch tensors q, k, v, out, dout against d."""
    import torch
    shapes = {"q": (d.batch, d.seqlen_q, d.num_heads_q, d.head_dim),
              "k": (d.batch, d.seqlen_k, d.num_heads_kv, d.head_dim),
              "v": (d.batch, d.seqlen_k, d.num_heads_kv, d.head_dim),
              "out": (d.batch, d.seqlen_q, d.num_heads_q, d.head_dim),
              "dout": (d.batch, d.seqlen_q, d.num_heads_q, d.head_dim),
              "q_idx": (d.batch, d.seqlen_q, d.num_heads_kv, d.index_dim),
              "k_idx": (d.batch, d.seqlen_k, d.index_dim)}
    for n, t in ts.items():
        _expect(n, t, torch.bfloat16, shapes[n], dev)


def _selection(d, dev, block_idx):
    import torch
    _expect("block_idx", block_idx, torch.int32, (d.batch, d.num_heads_kv, d.seqlen_q, d.topk), dev)


def _lse(d, dev, name, t):
    import torch
    _expect(name, t, torch.float32, (d.batch, d.num_heads_q, d.seqlen_q), dev)


def _workspace(dims, entry, ws, dev):
    import torch
    if ws is None:
        need = msa_workspace_bytes(dims, entry)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    else:
        if not (isinstance(ws, torch.Tensor) and ws.is_contiguous() and ws.is_cuda and ws.device == dev):
            raise ValueError("workspace must be a contiguous CUDA tensor on the arguments' device")
    return ws, ws.numel() * ws.element_size()


# ------------------------------------------------------------ entry points
def msa_index_scores(q_idx, k_idx, *, block_size=128, topk=16, block_scores=None):
    """Block scores [B, H_kv, S_q, n_blk] fp32 of the index branch."""
    import torch
    d = dims_of(q_idx=q_idx, k_idx=k_idx, topk=topk, block_size=block_size)
    dev = q_idx.device
    _main_inputs(d, dev, q_idx=q_idx, k_idx=k_idx)
    block_scores = _out("block_scores", block_scores, torch.float32,
                        (d.batch, d.num_heads_kv, d.seqlen_q, d.n_blk), dev)
    rc = lib().msa_index_scores(ctypes.byref(d), _ptr(q_idx), _ptr(k_idx), _ptr(block_scores), _stream(dev))
    _check(rc, "msa_index_scores")
    return block_scores


def _selection_dims(B, Hkv, Sq, seqlen_k, topk, block_size):
    return Dims.make(B, Sq, seqlen_k, Hkv, Hkv, 128, 128, block_size, topk, 1, 0.0)


def msa_block_topk(block_scores, *, seqlen_k, topk=16, block_size=128, block_idx=None):
    """Selected blocks [B, H_kv, S_q, topk] int32 (ascending, -1 padded)."""
    import torch
    _rank("block_scores", block_scores, 4)
    B, Hkv, Sq, _ = block_scores.shape
    d = _selection_dims(B, Hkv, Sq, seqlen_k, topk, block_size)
    dev = block_scores.device
    _expect("block_scores", block_scores, torch.float32, (B, Hkv, Sq, d.n_blk), dev)
    block_idx = _out("block_idx", block_idx, torch.int32, (B, Hkv, Sq, topk), dev)
    rc = lib().msa_block_topk(ctypes.byref(d), _ptr(block_scores), _ptr(block_idx), _stream(dev))
    _check(rc, "msa_block_topk")
    return block_idx


def msa_block_mask(block_idx, *, seqlen_k, block_size=128, mask=None):
    """Block-mask form [B, H_kv, S_q, ceil(n_blk / 32)] (int32 tensor holding
    uint32 words) of a selection [B, H_kv, S_q, topk]."""
    import torch
    _rank("block_idx", block_idx, 4)
    B, Hkv, Sq, topk = block_idx.shape
    d = _selection_dims(B, Hkv, Sq, seqlen_k, topk, block_size)
    dev = block_idx.device
    _selection(d, dev, block_idx)
    mask = _out("mask", mask, torch.int32, (B, Hkv, Sq, -(-d.n_blk // 32)), dev)
    rc = lib().msa_block_mask(ctypes.byref(d), _ptr(block_idx), _ptr(mask), _stream(dev))
    _check(rc, "msa_block_mask")
    return mask


def msa_mask_blocks(mask, *, seqlen_k, topk=16, block_size=128, block_idx=None):
    """Traversal of block masks [B, H_kv, S_q, n_words]: the set blocks in
    ascending order, at most topk per row, -1 padded -> [B, H_kv, S_q, topk]."""
    import torch
    _rank("mask", mask, 4)
    B, Hkv, Sq, _ = mask.shape
    d = _selection_dims(B, Hkv, Sq, seqlen_k, topk, block_size)
    dev = mask.device
    _expect("mask", mask, torch.int32, (B, Hkv, Sq, -(-d.n_blk // 32)), dev)
    block_idx = _out("block_idx", block_idx, torch.int32, (B, Hkv, Sq, topk), dev)
    rc = lib().msa_mask_blocks(ctypes.byref(d), _ptr(mask), _ptr(block_idx), _stream(dev))
    _check(rc, "msa_mask_blocks")
    return block_idx


def msa_sparse_attn_fwd(q, k, v, block_idx, *, block_size=128, softmax_scale=0.0, out=None,
                        return_lse=False, lse=None, workspace=None):
    """Main-branch attention over the selected blocks; returns out (and lse
    when return_lse is set or an lse tensor is passed)."""
    import torch
    _rank("block_idx", block_idx, 4)
    d = dims_of(q, k, topk=block_idx.shape[-1], block_size=block_size, softmax_scale=softmax_scale)
    dev = q.device
    _main_inputs(d, dev, q=q, k=k, v=v)
    _selection(d, dev, block_idx)
    out = _out("out", out, torch.bfloat16, tuple(q.shape), dev)
    want_lse = return_lse or lse is not None
    if want_lse:
        lse = _out("lse", lse, torch.float32, (d.batch, d.num_heads_q, d.seqlen_q), dev)
    ws, nbytes = _workspace(d, ENTRY_SPARSE_ATTN_FWD, workspace, dev)
    rc = lib().msa_sparse_attn_fwd(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(block_idx),
                                   _ptr(out), _ptr(lse), _ptr(ws), nbytes, _stream(dev))
    _check(rc, "msa_sparse_attn_fwd")
    return (out, lse) if want_lse else out


def msa_forward(q, k, v, q_idx, k_idx, *, topk=16, block_size=128, softmax_scale=0.0, out=None,
                lse=None, block_idx=None, return_lse=False, return_idx=False, workspace=None,
                stage_events=None):
    """Index scores -> Top-k -> sparse attention.  Returns out, plus lse and
    block_idx when asked (return_lse / return_idx, or a tensor passed for
    them).  stage_events: raw hipEvent_t handles for msa_forward_profiled,
    n_stage_events(chunks) of them."""
    import torch
    d = dims_of(q, k, q_idx, k_idx, topk=topk, block_size=block_size, softmax_scale=softmax_scale)
    dev = q.device
    _main_inputs(d, dev, q=q, k=k, v=v, q_idx=q_idx, k_idx=k_idx)
    out = _out("out", out, torch.bfloat16, tuple(q.shape), dev)
    want_lse, want_idx = return_lse or lse is not None, return_idx or block_idx is not None
    if want_lse:
        lse = _out("lse", lse, torch.float32, (d.batch, d.num_heads_q, d.seqlen_q), dev)
    if want_idx:
        block_idx = _out("block_idx", block_idx, torch.int32, (d.batch, d.num_heads_kv, d.seqlen_q, topk), dev)
    ws, nbytes = _workspace(d, ENTRY_FORWARD, workspace, dev)
    args = (ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(q_idx), _ptr(k_idx), _ptr(out),
            _ptr(lse if want_lse else None), _ptr(block_idx if want_idx else None), _ptr(ws), nbytes,
            _stream(dev))
    if stage_events is None:
        rc = lib().msa_forward(*args)
        _check(rc, "msa_forward")
    else:
        arr = (ctypes.c_void_p * len(stage_events))(*stage_events)
        rc = lib().msa_forward_profiled(*args, arr, len(stage_events))
        _check(rc, "msa_forward_profiled")
    res = [out]
    if want_lse:
        res.append(lse)
    if want_idx:
        res.append(block_idx)
    return res[0] if len(res) == 1 else tuple(res)


def msa_forward_noalloc(q, k, v, q_idx, k_idx, *, topk=16, block_size=128, softmax_scale=0.0, out=None,
                        lse=None, block_idx=None, return_lse=False, return_idx=False):
    """msa_forward on the library's static scratch instead of a caller
    workspace (the C entry point allocates nothing; outputs not passed in are
    allocated here, before the call).  Returns as msa_forward."""
    import torch
    d = dims_of(q, k, q_idx, k_idx, topk=topk, block_size=block_size, softmax_scale=softmax_scale)
    dev = q.device
    _main_inputs(d, dev, q=q, k=k, v=v, q_idx=q_idx, k_idx=k_idx)
    out = _out("out", out, torch.bfloat16, tuple(q.shape), dev)
    want_lse, want_idx = return_lse or lse is not None, return_idx or block_idx is not None
    if want_lse:
        lse = _out("lse", lse, torch.float32, (d.batch, d.num_heads_q, d.seqlen_q), dev)
    if want_idx:
        block_idx = _out("block_idx", block_idx, torch.int32, (d.batch, d.num_heads_kv, d.seqlen_q, topk), dev)
    rc = lib().msa_forward_noalloc(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(q_idx), _ptr(k_idx), _ptr(out),
                                   _ptr(lse if want_lse else None), _ptr(block_idx if want_idx else None),
                                   _stream(dev))
    _check(rc, "msa_forward_noalloc")
    res = [out] + ([lse] if want_lse else []) + ([block_idx] if want_idx else [])
    return res[0] if len(res) == 1 else tuple(res)


def default_softmax_scale(head_dim: int = 128) -> float:
    return 1.0 / math.sqrt(head_dim)


def msa_kl_loss_fwd(q, k, q_idx, k_idx, block_idx, lse, *, block_size=128, softmax_scale=0.0,
                    return_rows=False, return_lse_idx=False, loss=None, rows=None, lse_idx=None,
                    workspace=None):
    """Alignment loss of the index branch (forward value): the mean over
    (batch, query, group) rows of KL(group-mean main-branch probabilities ||
    softmax of the index scores) on each row's selected tokens.  ``lse`` is
    the main branch's log-sum-exp over the same selection ([B, H_q, S_q], as
    msa_forward returns it).  Returns the loss as a 0-d fp32 tensor, then the
    per-row terms [B, H_kv, S_q] when return_rows is set (or rows is passed)
    and the rows' log-sum-exps of the index scores [B, H_kv, S_q] when
    return_lse_idx is set (or lse_idx is passed)."""
    import torch
    _rank("block_idx", block_idx, 4)
    d = dims_of(q, k, q_idx, k_idx, topk=block_idx.shape[-1], block_size=block_size,
                softmax_scale=softmax_scale)
    dev = q.device
    _main_inputs(d, dev, q=q, k=k, q_idx=q_idx, k_idx=k_idx)
    _selection(d, dev, block_idx)
    _lse(d, dev, "lse", lse)
    shape = (d.batch, d.num_heads_kv, d.seqlen_q)
    want_rows, want_li = return_rows or rows is not None, return_lse_idx or lse_idx is not None
    loss = _out("loss", loss, torch.float32, (), dev)
    rows = _out("rows", rows, torch.float32, shape, dev) if want_rows else None
    lse_idx = _out("lse_idx", lse_idx, torch.float32, shape, dev) if want_li else None
    ws, nbytes = _workspace(d, ENTRY_KL_LOSS_FWD, workspace, dev)
    rc = lib().msa_kl_loss_fwd(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(q_idx), _ptr(k_idx),
                               _ptr(block_idx), _ptr(lse), _ptr(rows), _ptr(loss), _ptr(lse_idx), _ptr(ws),
                               nbytes, _stream(dev))
    _check(rc, "msa_kl_loss_fwd")
    res = [loss] + ([rows] if want_rows else []) + ([lse_idx] if want_li else [])
    return res[0] if len(res) == 1 else tuple(res)


def msa_sparse_attn_bwd(q, k, v, block_idx, out, lse, dout, *, block_size=128, softmax_scale=0.0,
                        dq=None, dk=None, dv=None, workspace=None):
    """Main-branch backward over the selection: returns (dq, dk, dv), bf16,
    from the upstream gradient dout and the forward's out and lse."""
    import torch
    _rank("block_idx", block_idx, 4)
    d = dims_of(q, k, topk=block_idx.shape[-1], block_size=block_size, softmax_scale=softmax_scale)
    dev = q.device
    _main_inputs(d, dev, q=q, k=k, v=v, out=out, dout=dout)
    _selection(d, dev, block_idx)
    _lse(d, dev, "lse", lse)
    dq = _out("dq", dq, torch.bfloat16, tuple(q.shape), dev)
    dk = _out("dk", dk, torch.bfloat16, tuple(k.shape), dev)
    dv = _out("dv", dv, torch.bfloat16, tuple(v.shape), dev)
    ws, nbytes = _workspace(d, ENTRY_SPARSE_ATTN_BWD, workspace, dev)
    rc = lib().msa_sparse_attn_bwd(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(block_idx), _ptr(out),
                                   _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), nbytes,
                                   _stream(dev))
    _check(rc, "msa_sparse_attn_bwd")
    return dq, dk, dv


def msa_backward(q, k, v, q_idx, k_idx, block_idx, out, lse, lse_idx, dout, grad_loss=1.0, *, block_size=128,
                 softmax_scale=0.0, dq=None, dk=None, dv=None, dq_idx=None, dk_idx=None, workspace=None):
    """Both backward passes in one call: returns (dq, dk, dv, dq_idx, dk_idx),
    bf16, equal bit for bit to msa_sparse_attn_bwd's and msa_kl_loss_bwd's
    outputs when each call runs in one query chunk."""
    import torch
    _rank("block_idx", block_idx, 4)
    d = dims_of(q, k, q_idx, k_idx, topk=block_idx.shape[-1], block_size=block_size,
                softmax_scale=softmax_scale)
    dev = q.device
    _main_inputs(d, dev, q=q, k=k, v=v, q_idx=q_idx, k_idx=k_idx, out=out, dout=dout)
    _selection(d, dev, block_idx)
    _lse(d, dev, "lse", lse)
    _expect("lse_idx", lse_idx, torch.float32, (d.batch, d.num_heads_kv, d.seqlen_q), dev)
    dq = _out("dq", dq, torch.bfloat16, tuple(q.shape), dev)
    dk = _out("dk", dk, torch.bfloat16, tuple(k.shape), dev)
    dv = _out("dv", dv, torch.bfloat16, tuple(v.shape), dev)
    dq_idx = _out("dq_idx", dq_idx, torch.bfloat16, tuple(q_idx.shape), dev)
    dk_idx = _out("dk_idx", dk_idx, torch.bfloat16, tuple(k_idx.shape), dev)
    ws, nbytes = _workspace(d, ENTRY_BACKWARD, workspace, dev)
    rc = lib().msa_backward(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(q_idx), _ptr(k_idx), _ptr(block_idx),
                            _ptr(out), _ptr(lse), _ptr(lse_idx), _ptr(dout), float(grad_loss), _ptr(dq), _ptr(dk),
                            _ptr(dv), _ptr(dq_idx), _ptr(dk_idx), _ptr(ws), nbytes, _stream(dev))
    _check(rc, "msa_backward")
    return dq, dk, dv, dq_idx, dk_idx


def msa_kl_loss_bwd(q, k, q_idx, k_idx, block_idx, lse, lse_idx, grad_loss=1.0, *, block_size=128,
                    softmax_scale=0.0, dq_idx=None, dk_idx=None, workspace=None):
    """Gradient of grad_loss * (the alignment loss) with respect to q_idx and
    k_idx, the teacher detached: returns (dq_idx, dk_idx), bf16.  lse is the
    main branch's LSE and lse_idx the index scores' LSE of msa_kl_loss_fwd."""
    import torch
    _rank("block_idx", block_idx, 4)
    d = dims_of(q, k, q_idx, k_idx, topk=block_idx.shape[-1], block_size=block_size,
                softmax_scale=softmax_scale)
    dev = q.device
    _main_inputs(d, dev, q=q, k=k, q_idx=q_idx, k_idx=k_idx)
    _selection(d, dev, block_idx)
    _lse(d, dev, "lse", lse)
    _expect("lse_idx", lse_idx, torch.float32, (d.batch, d.num_heads_kv, d.seqlen_q), dev)
    dq_idx = _out("dq_idx", dq_idx, torch.bfloat16, tuple(q_idx.shape), dev)
    dk_idx = _out("dk_idx", dk_idx, torch.bfloat16, tuple(k_idx.shape), dev)
    ws, nbytes = _workspace(d, ENTRY_KL_LOSS_BWD, workspace, dev)
    rc = lib().msa_kl_loss_bwd(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(q_idx), _ptr(k_idx), _ptr(block_idx),
                               _ptr(lse), _ptr(lse_idx), float(grad_loss), _ptr(dq_idx), _ptr(dk_idx), _ptr(ws),
                               nbytes, _stream(dev))
    _check(rc, "msa_kl_loss_bwd")
    return dq_idx, dk_idx

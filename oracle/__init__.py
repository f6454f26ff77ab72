"""Python access to the CPU oracle of the MSA forward path.

TEST INFRASTRUCTURE ONLY.  The oracle is a plain, slow fp64 restatement of
the method (see ``msa_oracle.cpp`` for the passages it follows).  Only the
tests, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline`` leg
may import this module; the device library never does.

Inputs are numpy arrays of bf16 bit patterns (uint16) in the library's
layouts.  ``rows`` lists the (b, i, g) triples to compute.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")


class _Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "batch", "seqlen_q", "seqlen_k", "heads_q", "heads_kv", "head_dim",
        "index_dim", "block_size", "topk")] + [("softmax_scale", ctypes.c_double)]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _b
            _b.build()
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        lib.oracle_block_scores.argtypes = [P, P, P, P, ctypes.c_int64, P, ctypes.c_int]
        lib.oracle_select.argtypes = [P, P, ctypes.c_int64, P, P]
        lib.oracle_attention.argtypes = [P, P, P, P, P, ctypes.c_int64, P, P, P, ctypes.c_int]
        lib.oracle_forward.argtypes = [P, P, P, P, P, P, P, ctypes.c_int64, P, P, P, P, ctypes.c_int]
        lib.oracle_kl_rows.argtypes = [P, P, P, P, P, P, ctypes.c_int64, P, P, ctypes.c_int]
        lib.oracle_kl_rows_f64.argtypes = lib.oracle_kl_rows.argtypes
        lib.oracle_attention_f64.argtypes = lib.oracle_attention.argtypes
        lib.oracle_attention_bwd.argtypes = [P, P, P, P, P, P, ctypes.c_int64, P, P, P, P, ctypes.c_int]
        lib.oracle_attention_bwd_f64.argtypes = lib.oracle_attention_bwd.argtypes
        lib.oracle_kl_bwd.argtypes = [P, P, P, P, P, P, ctypes.c_int64, P, P, P, P, ctypes.c_int]
        lib.oracle_kl_bwd_f64.argtypes = lib.oracle_kl_bwd.argtypes
        for f in (lib.oracle_block_scores, lib.oracle_select, lib.oracle_attention,
                  lib.oracle_forward, lib.oracle_kl_rows, lib.oracle_default_threads,
                  lib.oracle_kl_rows_f64, lib.oracle_attention_f64, lib.oracle_attention_bwd,
                  lib.oracle_attention_bwd_f64, lib.oracle_kl_bwd, lib.oracle_kl_bwd_f64):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads() -> int:
    """Worker threads used when a call passes threads=0: every core, capped by
    OMP_NUM_THREADS when that is set."""
    n = _load().oracle_default_threads()
    cap = os.environ.get("OMP_NUM_THREADS", "")
    return min(n, int(cap)) if cap.isdigit() and int(cap) > 0 else n


class Problem:
    """Shapes of one problem, as the oracle sees them."""

    def __init__(self, batch, seqlen_q, seqlen_k, heads_q, heads_kv, head_dim,
                 index_dim, block_size=128, topk=16, softmax_scale=0.0):
        self.batch, self.seqlen_q, self.seqlen_k = batch, seqlen_q, seqlen_k
        self.heads_q, self.heads_kv, self.head_dim = heads_q, heads_kv, head_dim
        self.index_dim, self.block_size, self.topk = index_dim, block_size, topk
        self.softmax_scale = softmax_scale

    @classmethod
    def of(cls, w, **kw):
        """From a ``synth.Workload`` (or anything with the same fields)."""
        args = dict(batch=w.batch, seqlen_q=w.seqlen_q, seqlen_k=w.seqlen_k, heads_q=w.heads_q,
                    heads_kv=w.heads_kv, head_dim=w.head_dim, index_dim=w.index_dim,
                    block_size=w.block_size, topk=w.topk)
        args.update(kw)
        return cls(**args)

    @property
    def n_blk(self):
        return -(-self.seqlen_k // self.block_size)

    @property
    def group(self):
        return self.heads_q // self.heads_kv

    def _c(self):
        return _Dims(self.batch, self.seqlen_q, self.seqlen_k, self.heads_q, self.heads_kv,
                     self.head_dim, self.index_dim, self.block_size, self.topk,
                     float(self.softmax_scale))

    def all_rows(self):
        b, i, g = np.meshgrid(np.arange(self.batch), np.arange(self.seqlen_q),
                              np.arange(self.heads_kv), indexing="ij")
        return np.stack([b.ravel(), i.ravel(), g.ravel()], axis=1).astype(np.int64)


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data)


def _u16(a, shape):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("oracle inputs are bf16 bit patterns (uint16)")
    if tuple(a.shape) != tuple(shape):
        raise ValueError(f"shape {a.shape} != {shape}")
    return a


def _inputs(arrays_shapes):
    """bf16 bit patterns (uint16) or fp64 values, all of one kind; returns
    (contiguous arrays, True when fp64)."""
    f64 = all(np.asarray(a).dtype == np.float64 for a, _ in arrays_shapes)
    out = []
    for a, shape in arrays_shapes:
        if f64:
            a = np.ascontiguousarray(a, dtype=np.float64)
            if tuple(a.shape) != tuple(shape):
                raise ValueError(f"shape {a.shape} != {shape}")
            out.append(a)
        else:
            out.append(_u16(a, shape))
    return out, f64


def _rows(p, rows):
    rows = p.all_rows() if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    return rows.reshape(-1, 3)


def block_scores(p: Problem, q_idx, k_idx, rows=None, threads=0):
    rows = _rows(p, rows)
    qi = _u16(q_idx, (p.batch, p.seqlen_q, p.heads_kv, p.index_dim))
    ki = _u16(k_idx, (p.batch, p.seqlen_k, p.index_dim))
    bm = np.empty((len(rows), p.n_blk), dtype=np.float64)
    d = p._c()
    rc = _load().oracle_block_scores(ctypes.byref(d), _ptr(qi), _ptr(ki), _ptr(rows), len(rows),
                                     _ptr(bm), threads or default_threads())
    if rc:
        raise ValueError("oracle_block_scores rejected its arguments")
    return bm


def select(p: Problem, bm, rows=None):
    rows = _rows(p, rows)
    bm = np.ascontiguousarray(bm, dtype=np.float64).reshape(len(rows), p.n_blk)
    sel = np.empty((len(rows), p.topk), dtype=np.int32)
    d = p._c()
    rc = _load().oracle_select(ctypes.byref(d), _ptr(rows), len(rows), _ptr(bm), _ptr(sel))
    if rc:
        raise ValueError("oracle_select rejected its arguments")
    return sel


def attention(p: Problem, q, k, v, sel, rows=None, threads=0):
    rows = _rows(p, rows)
    (qq, kk, vv), f64 = _inputs([(q, (p.batch, p.seqlen_q, p.heads_q, p.head_dim)),
                                 (k, (p.batch, p.seqlen_k, p.heads_kv, p.head_dim)),
                                 (v, (p.batch, p.seqlen_k, p.heads_kv, p.head_dim))])
    sel = np.ascontiguousarray(sel, dtype=np.int32).reshape(len(rows), p.topk)
    out = np.empty((len(rows), p.group, p.head_dim), dtype=np.float64)
    lse = np.empty((len(rows), p.group), dtype=np.float64)
    d = p._c()
    fn = _load().oracle_attention_f64 if f64 else _load().oracle_attention
    rc = fn(ctypes.byref(d), _ptr(qq), _ptr(kk), _ptr(vv), _ptr(rows),
            len(rows), _ptr(sel), _ptr(out), _ptr(lse), threads or default_threads())
    if rc:
        raise ValueError("oracle_attention rejected its arguments")
    return out, lse


def forward(p: Problem, q, k, v, q_idx, k_idx, rows=None, threads=0):
    """Block scores, selection, output and LSE for the listed rows."""
    rows = _rows(p, rows)
    qq = _u16(q, (p.batch, p.seqlen_q, p.heads_q, p.head_dim))
    kk = _u16(k, (p.batch, p.seqlen_k, p.heads_kv, p.head_dim))
    vv = _u16(v, (p.batch, p.seqlen_k, p.heads_kv, p.head_dim))
    qi = _u16(q_idx, (p.batch, p.seqlen_q, p.heads_kv, p.index_dim))
    ki = _u16(k_idx, (p.batch, p.seqlen_k, p.index_dim))
    n = len(rows)
    bm = np.empty((n, p.n_blk), dtype=np.float64)
    sel = np.empty((n, p.topk), dtype=np.int32)
    out = np.empty((n, p.group, p.head_dim), dtype=np.float64)
    lse = np.empty((n, p.group), dtype=np.float64)
    d = p._c()
    rc = _load().oracle_forward(ctypes.byref(d), _ptr(qq), _ptr(kk), _ptr(vv), _ptr(qi), _ptr(ki),
                                _ptr(rows), n, _ptr(bm), _ptr(sel), _ptr(out), _ptr(lse), threads or default_threads())
    if rc:
        raise ValueError("oracle_forward rejected its arguments")
    return {"bm": bm, "sel": sel, "out": out, "lse": lse, "rows": rows}


def kl_rows(p: Problem, q, k, q_idx, k_idx, sel, rows=None, threads=0):
    """KL-alignment loss term of each listed row (Sparse Attention Part II,
    section 3.2): KL(teacher || student) over the row's selected visible
    tokens, teacher = the group's mean per-head attention probabilities,
    student = softmax of the raw index scores.  The loss is the mean over
    all N * H_kv rows."""
    rows = _rows(p, rows)
    (qq, kk, qi, ki), f64 = _inputs(_kl_shapes(p, q, k, q_idx, k_idx))
    sel = np.ascontiguousarray(sel, dtype=np.int32).reshape(len(rows), p.topk)
    kl = np.empty(len(rows), dtype=np.float64)
    d = p._c()
    fn = _load().oracle_kl_rows_f64 if f64 else _load().oracle_kl_rows
    rc = fn(ctypes.byref(d), _ptr(qq), _ptr(kk), _ptr(qi), _ptr(ki), _ptr(rows),
            len(rows), _ptr(sel), _ptr(kl), threads or default_threads())
    if rc:
        raise ValueError("oracle_kl_rows rejected its arguments")
    return kl


def _kl_shapes(p, q, k, q_idx, k_idx):
    return [(q, (p.batch, p.seqlen_q, p.heads_q, p.head_dim)),
            (k, (p.batch, p.seqlen_k, p.heads_kv, p.head_dim)),
            (q_idx, (p.batch, p.seqlen_q, p.heads_kv, p.index_dim)),
            (k_idx, (p.batch, p.seqlen_k, p.index_dim))]


def attention_bwd(p: Problem, q, k, v, dout, sel, rows=None, threads=0, want_dkv=True):
    """Gradient of the main branch given dO (same layout as q): dq of each
    listed row [n_rows, G, D], and dk, dv [B, S_k, H_kv, D] summed over the
    listed rows (None when want_dkv is False).  The selection carries no
    gradient; inside it the attention is a softmax attention over the
    selected visible tokens."""
    rows = _rows(p, rows)
    (qq, kk, vv, do), f64 = _inputs([(q, (p.batch, p.seqlen_q, p.heads_q, p.head_dim)),
                                     (k, (p.batch, p.seqlen_k, p.heads_kv, p.head_dim)),
                                     (v, (p.batch, p.seqlen_k, p.heads_kv, p.head_dim)),
                                     (dout, (p.batch, p.seqlen_q, p.heads_q, p.head_dim))])
    sel = np.ascontiguousarray(sel, dtype=np.int32).reshape(len(rows), p.topk)
    dq = np.empty((len(rows), p.group, p.head_dim), dtype=np.float64)
    dk = np.empty((p.batch, p.seqlen_k, p.heads_kv, p.head_dim), dtype=np.float64) if want_dkv else None
    dv = np.empty_like(dk) if want_dkv else None
    d = p._c()
    fn = _load().oracle_attention_bwd_f64 if f64 else _load().oracle_attention_bwd
    rc = fn(ctypes.byref(d), _ptr(qq), _ptr(kk), _ptr(vv), _ptr(do), _ptr(rows), len(rows), _ptr(sel),
            _ptr(dq), None if dk is None else _ptr(dk), None if dv is None else _ptr(dv),
            threads or default_threads())
    if rc:
        raise ValueError("oracle_attention_bwd rejected its arguments")
    return dq, dk, dv


def kl_bwd(p: Problem, q, k, q_idx, k_idx, sel, rows=None, threads=0, want_dk=True):
    """Gradient of the listed rows' KL terms with respect to the index
    inputs, the teacher held fixed (section 3.2 detaches it): dq_idx of each
    row [n_rows, D_idx], dk_idx [B, S_k, D_idx] summed over the rows, and each
    row's log-sum-exp of the index scores over its tokens.  Unscaled: the
    loss's 1 / (N H_kv) is the caller's."""
    rows = _rows(p, rows)
    (qq, kk, qi, ki), f64 = _inputs(_kl_shapes(p, q, k, q_idx, k_idx))
    sel = np.ascontiguousarray(sel, dtype=np.int32).reshape(len(rows), p.topk)
    dqi = np.empty((len(rows), p.index_dim), dtype=np.float64)
    dki = np.empty((p.batch, p.seqlen_k, p.index_dim), dtype=np.float64) if want_dk else None
    lse_z = np.empty(len(rows), dtype=np.float64)
    d = p._c()
    fn = _load().oracle_kl_bwd_f64 if f64 else _load().oracle_kl_bwd
    rc = fn(ctypes.byref(d), _ptr(qq), _ptr(kk), _ptr(qi), _ptr(ki), _ptr(rows), len(rows), _ptr(sel),
            _ptr(dqi), None if dki is None else _ptr(dki), _ptr(lse_z), threads or default_threads())
    if rc:
        raise ValueError("oracle_kl_bwd rejected its arguments")
    return dqi, dki, lse_z


# ------------------------------------------------- block-mask selection format
# Sparse Attention Part II, section 4.3: the blocks a query (block) visits are
# flags packed 32 to an unsigned word; block j is bit j mod 32 of word
# floor(j / 32), set by OR-ing 1 << (j mod 32) into that word.  A traversal
# walks the words, takes each word's popcount as its number of active blocks
# and the rank-th set bit (nth_set_bit) as the position of the rank-th one.
# Bits past the last block stay zero.  Storage: 4 * ceil(n_blk / 32) bytes per
# row, i.e. 4 T_r ceil(T_c / 32) per batch item and head for T_r row blocks.

def mask_words(n_blk: int) -> int:
    """32-bit words per row of a mask over n_blk blocks."""
    return -(-n_blk // 32)


def block_mask(sel, n_blk: int):
    """Selections [..., k] (block indices, -1 = unused) -> masks
    [..., ceil(n_blk / 32)] uint32, bit j mod 32 of word j // 32 per block j."""
    sel = np.asarray(sel)
    flat = sel.reshape(-1, sel.shape[-1]).astype(np.int64)
    mask = np.zeros((flat.shape[0], mask_words(n_blk)), dtype=np.uint32)
    r, e = np.nonzero((flat >= 0) & (flat < n_blk))
    j = flat[r, e]
    np.bitwise_or.at(mask, (r, j // 32), np.left_shift(np.uint32(1), (j % 32).astype(np.uint32)))
    return mask.reshape(sel.shape[:-1] + (mask.shape[-1],))


def popcount(word: int) -> int:
    """Number of set bits of a 32-bit word."""
    return sum((int(word) >> b) & 1 for b in range(32))


def nth_set_bit(word: int, rank: int) -> int:
    """Position of the rank-th (zero-based) set bit of a 32-bit word."""
    seen = 0
    for b in range(32):
        if (int(word) >> b) & 1:
            if seen == rank:
                return b
            seen += 1
    raise ValueError("rank past the word's popcount")


def mask_blocks(mask, cap: int):
    """Masks [..., n_words] -> block lists [..., cap] int32: the set bits in
    ascending block order (the traversal order), at most cap of them (the
    lowest), padded with -1."""
    mask = np.asarray(mask, dtype=np.uint32)
    flat = mask.reshape(-1, mask.shape[-1])
    n_rows, n_words = flat.shape
    bits = (flat[:, :, None] >> np.arange(32, dtype=np.uint32)[None, None, :]) & 1  # [rows, words, 32]
    on = bits.reshape(n_rows, n_words * 32).astype(bool)  # position 32 w + b, ascending
    out = np.full((n_rows, cap), -1, dtype=np.int32)
    r, j = np.nonzero(on)  # row-major: ascending j within each row
    rank = np.arange(len(r)) - np.searchsorted(r, r)  # position of each set bit within its row
    keep = rank < cap
    out[r[keep], rank[keep]] = j[keep]
    return out.reshape(mask.shape[:-1] + (cap,))


def mask_blocks_by_scan(mask_row, n_blk: int, cap: int):
    """One row from the bit-set definition alone: block j is in the row when
    bit j mod 32 of word floor(j / 32) is set; scanning j = 0 .. n_blk-1 in
    order keeps the first cap of them.  Pure Python, for small cases."""
    words = [int(x) for x in np.asarray(mask_row, dtype=np.uint32).tolist()]
    out = [j for j in range(n_blk) if (words[j // 32] >> (j % 32)) & 1][:cap]
    return out + [-1] * (cap - len(out))

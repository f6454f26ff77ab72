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
        for f in (lib.oracle_block_scores, lib.oracle_select, lib.oracle_attention,
                  lib.oracle_forward, lib.oracle_default_threads):
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
    qq = _u16(q, (p.batch, p.seqlen_q, p.heads_q, p.head_dim))
    kk = _u16(k, (p.batch, p.seqlen_k, p.heads_kv, p.head_dim))
    vv = _u16(v, (p.batch, p.seqlen_k, p.heads_kv, p.head_dim))
    sel = np.ascontiguousarray(sel, dtype=np.int32).reshape(len(rows), p.topk)
    out = np.empty((len(rows), p.group, p.head_dim), dtype=np.float64)
    lse = np.empty((len(rows), p.group), dtype=np.float64)
    d = p._c()
    rc = _load().oracle_attention(ctypes.byref(d), _ptr(qq), _ptr(kk), _ptr(vv), _ptr(rows),
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

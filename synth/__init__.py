"""Seeded synthetic inputs shared by the oracle side and the device side.

This module holds no part of the attention method.  It defines the workloads
(shapes and value distributions) and one counter-based generator, implemented
twice from its published definition: here on the host with numpy, and in
``synth_fill.hip`` on the device.  Tests and the benchmark draw every input
from it; the oracle and the device library each receive the same tensors.

Generator definition
--------------------
* counter(e) = seed XOR (tensor_id << 40) XOR e, for element e of the tensor
  in row-major order;
* x = splitmix64(counter) (Steele, Lea and Flood, OOPSLA 2014);
* u(e) = (x >> 11) * 2**-53, uniform in [0, 1);
* integers: floor(7 u) - 3, uniform in {-3, ..., 3};
* normals: Box-Muller on the element pair (2m, 2m+1) with m = e >> 1:
  r = sqrt(-2 ln(1 - u(2m))), th = 2 pi u(2m+1); r cos th for even e, r sin th
  for odd e (float64);
* stored as bf16: the float64 value is rounded to float32, then to bf16, both
  round-to-nearest-even;
* optional per-block gain g_j = exp(0.5 * normal_6(j)) for key block j
  (tensor id 6): a normal element becomes g_j * z before rounding; an integer
  element becomes rint_half_even(g_j * n), still an exact bf16 integer.

Tensor ids: Q 1, K 2, V 3, Q_idx 4, K_idx 5, gain 6, dO 7 (the upstream gradient
of the output, for the backward).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, replace

import numpy as np

TENSOR_IDS = {"q": 1, "k": 2, "v": 3, "q_idx": 4, "k_idx": 5, "gain": 6, "dout": 7}
_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmsa_synth.so")

_M64 = np.uint64(0xFFFFFFFFFFFFFFFF)


# ---------------------------------------------------------------- workloads
@dataclass(frozen=True)
class Workload:
    """One synthetic problem: shapes, selection parameters and distributions.

    Index inputs (q_idx, k_idx) are integers uniform in [-3, 3] stored exactly
    in bf16, so every fp32 index score is an exact integer.  Q, K and V are
    N(0, 1) rounded to bf16.  With ``gain`` set, the K and k_idx rows of key
    block j are scaled by a LogNormal(0, 0.5) gain g_j (k_idx rounded back to
    integers), which makes block scores uneven across blocks.
    """

    name: str
    batch: int
    seqlen_q: int
    seqlen_k: int
    heads_q: int
    heads_kv: int
    head_dim: int = 128
    index_dim: int = 128
    block_size: int = 128
    topk: int = 16
    gain: bool = False
    seed: int = 0

    @property
    def n_blk(self) -> int:
        return -(-self.seqlen_k // self.block_size)

    @property
    def group(self) -> int:
        return self.heads_q // self.heads_kv

    def shapes(self) -> dict:
        B, Sq, Sk = self.batch, self.seqlen_q, self.seqlen_k
        return {
            "q": (B, Sq, self.heads_q, self.head_dim),
            "k": (B, Sk, self.heads_kv, self.head_dim),
            "v": (B, Sk, self.heads_kv, self.head_dim),
            "q_idx": (B, Sq, self.heads_kv, self.index_dim),
            "k_idx": (B, Sk, self.index_dim),
            "dout": (B, Sq, self.heads_q, self.head_dim),
        }

    def kind(self, name: str) -> str:
        return "int" if name in ("q_idx", "k_idx") else "normal"

    def gained(self, name: str) -> bool:
        return self.gain and name in ("k", "k_idx")

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads: 4K prefill (8/2 heads, index dim 64); 32K prefill;
# 128K prefill with uneven block gains; 64-sequence decode against a 256K-token
# cache; a 16K-query chunk at the end of a 1M-token prefix.
WORKLOADS = {
    "prefill_4k": Workload("prefill_4k", 1, 4096, 4096, 8, 2, index_dim=64),
    "prefill_32k": Workload("prefill_32k", 1, 32768, 32768, 64, 8),
    "prefill_128k_gain": Workload("prefill_128k_gain", 1, 131072, 131072, 64, 8, gain=True),
    "decode_64x256k": Workload("decode_64x256k", 64, 1, 262144, 64, 8),
    "chunk_16k_of_1m": Workload("chunk_16k_of_1m", 1, 16384, 1048576, 64, 8),
}


# ------------------------------------------------------------ host generator
def splitmix64(z: np.ndarray) -> np.ndarray:
    z = (z.astype(np.uint64) + np.uint64(0x9E3779B97F4A7C15)) & _M64
    z = ((z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)) & _M64
    z = ((z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)) & _M64
    return z ^ (z >> np.uint64(31))


def uniform(seed: int, tensor_id: int, e: np.ndarray) -> np.ndarray:
    c = np.uint64(seed) ^ (np.uint64(tensor_id) << np.uint64(40)) ^ np.asarray(e, dtype=np.uint64)
    x = splitmix64(c)
    return (x >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def normal(seed: int, tensor_id: int, e: np.ndarray) -> np.ndarray:
    e = np.asarray(e, dtype=np.uint64)
    m = e >> np.uint64(1)
    u1 = uniform(seed, tensor_id, m * np.uint64(2))
    u2 = uniform(seed, tensor_id, m * np.uint64(2) + np.uint64(1))
    r = np.sqrt(-2.0 * np.log(1.0 - u1))
    th = 2.0 * np.pi * u2
    return np.where((e & np.uint64(1)) == 1, r * np.sin(th), r * np.cos(th))


def integer(seed: int, tensor_id: int, e: np.ndarray) -> np.ndarray:
    return np.floor(7.0 * uniform(seed, tensor_id, e)) - 3.0


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))
    return (b >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def block_gain(seed: int, j: np.ndarray) -> np.ndarray:
    return np.exp(0.5 * normal(seed, TENSOR_IDS["gain"], j))


def values_f64(w: Workload, name: str, e: np.ndarray) -> np.ndarray:
    """Float64 value of elements ``e`` of tensor ``name`` before bf16 storage."""
    tid = TENSOR_IDS[name]
    e = np.asarray(e, dtype=np.uint64)
    if w.kind(name) == "int":
        v = integer(w.seed, tid, e)
    else:
        v = normal(w.seed, tid, e)
    if w.gained(name):
        per_tok = int(np.prod(w.shapes()[name][2:]))
        tok = (e // np.uint64(per_tok)) % np.uint64(w.seqlen_k)
        g = block_gain(w.seed, tok // np.uint64(w.block_size))
        v = np.rint(v * g) if w.kind(name) == "int" else v * g
    return v


def host_bits(w: Workload, name: str, e: np.ndarray) -> np.ndarray:
    """bf16 bits (uint16) of elements ``e`` of tensor ``name``."""
    return f32_to_bf16_bits(values_f64(w, name, e).astype(np.float32))


def host_tensor(w: Workload, name: str) -> np.ndarray:
    """The whole tensor as uint16 bf16 bits; for the small workloads only."""
    shape = w.shapes()[name]
    n = int(np.prod(shape))
    if n > (1 << 28):
        raise ValueError(f"{name} of {w.name} has {n} elements; draw it on the device")
    return host_bits(w, name, np.arange(n, dtype=np.uint64)).reshape(shape)


# ---------------------------------------------------------- device generator
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(LIB_PATH)
        for fn in (lib.synth_fill_normal_bf16, lib.synth_fill_int_bf16):
            fn.restype = ctypes.c_int
            fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32,
                           ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
        lib.synth_copy_bytes.restype = ctypes.c_int
        lib.synth_copy_bytes.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        _lib = lib
    return _lib


def copy_probe(nbytes: int, device="cuda", reps: int = 1) -> float:
    """Run ``reps`` plain device copies of ``nbytes`` (each reads and writes
    exactly that many bytes): the known-size reference for traffic counters.
    Returns the copy rate in GB/s (bytes read + written per second) over the
    reps after the first, or 0.0 when reps == 1."""
    import torch

    src = torch.empty(nbytes, dtype=torch.uint8, device=device)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream(src.device)
    lib = _load()

    def once():
        rc = lib.synth_copy_bytes(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                  nbytes, ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"copy probe failed ({rc})")

    once()
    if reps <= 1:
        torch.cuda.synchronize()
        return 0.0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps - 1):
        once()
    e1.record(stream)
    torch.cuda.synchronize()
    return 2.0 * nbytes * (reps - 1) / (e0.elapsed_time(e1) * 1e-3) / 1e9


def fill_device(w: Workload, name: str, tensor) -> None:
    """Fill a contiguous bf16 torch CUDA tensor with tensor ``name`` of ``w``."""
    import torch

    shape = w.shapes()[name]
    assert tuple(tensor.shape) == tuple(shape) and tensor.dtype == torch.bfloat16
    assert tensor.is_cuda and tensor.is_contiguous()
    lib = _load()
    fn = lib.synth_fill_int_bf16 if w.kind(name) == "int" else lib.synth_fill_normal_bf16
    per_tok = int(np.prod(shape[2:]))
    gain_block = w.block_size if w.gained(name) else 0
    stream = torch.cuda.current_stream(tensor.device).cuda_stream
    rc = fn(ctypes.c_void_p(tensor.data_ptr()), tensor.numel(), w.seed, TENSOR_IDS[name],
            per_tok, w.seqlen_k, gain_block, ctypes.c_void_p(stream))
    if rc != 0:
        raise RuntimeError(f"synth fill of {name} failed with HIP error {rc}")


def device_tensors(w: Workload, device="cuda", names=("q", "k", "v", "q_idx", "k_idx")) -> dict:
    """Allocate and fill the named inputs of ``w`` on ``device``."""
    import torch

    out = {}
    for name in names:
        t = torch.empty(w.shapes()[name], dtype=torch.bfloat16, device=device)
        fill_device(w, name, t)
        out[name] = t
    return out

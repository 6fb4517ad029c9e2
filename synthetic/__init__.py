"""Seeded synthetic inputs for the P-cast attention workloads.

This package produces input bytes only: bf16 Gaussian tensors from a
counter-based generator (``gen.c``) and the per-key sink bias vector.  It
holds none of the attention arithmetic, so the CPU oracle and the GPU path
can both draw identical inputs from it without sharing any of the method.

Sink bias: the first ``SINK_KEYS`` keys get an additive logit bias ``delta``
and every other key gets 0, which is the attention-sink setting of the P-cast
paper summary (section "Metodologia e Analisi": sink strength is the logit gap
between the k sink tokens and the rest, with k = 4).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

from .workloads import DECODE_WORKLOADS, WORKLOADS, DecodeWorkload, Workload  # noqa: F401

SINK_KEYS = 4
TENSOR_Q, TENSOR_K, TENSOR_V = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB = os.path.join(_HERE, "_gen.so")
_lock = threading.Lock()
_lib = None


def build() -> str:
    """Compile gen.c into _gen.so (always recompiles)."""
    tmp = _LIB + ".tmp"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"],
                   check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB):
                build()
            lib = ctypes.CDLL(_LIB)
            lib.synth_gaussian_bf16.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint64,
                                                ctypes.c_uint64, ctypes.c_void_p]
            lib.synth_gaussian_bf16.restype = None
            _lib = lib
    return _lib


def gaussian_bf16(seed: int, tensor_id: int, shape, first: int = 0) -> np.ndarray:
    """bf16 bit patterns (uint16) of i.i.d. N(0,1) draws, C-contiguous ``shape``.

    Element ``k`` of the flattened result is stream element ``first + k`` of
    stream (seed, tensor_id), so any slice of a large tensor can be produced
    without producing the rest.
    """
    n = int(np.prod(shape, dtype=np.int64))
    out = np.empty(n, dtype=np.uint16)
    if n:
        _load().synth_gaussian_bf16(seed, tensor_id, first, n, out.ctypes.data)
    return out.reshape(shape)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def sink_bias(n: int, delta: float, sink_keys: int = SINK_KEYS) -> np.ndarray:
    """float32 [n]: ``delta`` on keys 0..sink_keys-1, else 0."""
    b = np.zeros(n, dtype=np.float32)
    b[:min(sink_keys, n)] = np.float32(delta)
    return b


def random_bias(n: int, seed: int, zero_frac: float = 0.5, scale: float = 2.0) -> np.ndarray:
    """float32 [n]: N(0, scale^2) on a random subset of keys, exactly 0 on a
    fraction ``zero_frac`` of them (numpy's PCG64 stream seeded with ``seed``)."""
    rng = np.random.default_rng(seed)
    b = (rng.standard_normal(n) * scale).astype(np.float32)
    b[rng.random(n) < zero_frac] = 0.0
    return b


def qkv_bf16(B: int, Hq: int, Hkv: int, N: int, d: int, seed: int):
    """(Q, K, V) bf16 bit arrays shaped [B,Hq,N,d], [B,Hkv,N,d], [B,Hkv,N,d]."""
    q = gaussian_bf16(seed, TENSOR_Q, (B, Hq, N, d))
    k = gaussian_bf16(seed, TENSOR_K, (B, Hkv, N, d))
    v = gaussian_bf16(seed, TENSOR_V, (B, Hkv, N, d))
    return q, k, v


def decode_qkv_bf16(B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int, seed: int):
    """(Q, K, V) bf16 bit arrays for decode: [B,Hq,Nq,d], [B,Hkv,Nk,d], [B,Hkv,Nk,d]."""
    q = gaussian_bf16(seed, TENSOR_Q, (B, Hq, Nq, d))
    k = gaussian_bf16(seed, TENSOR_K, (B, Hkv, Nk, d))
    v = gaussian_bf16(seed, TENSOR_V, (B, Hkv, Nk, d))
    return q, k, v

"""ctypes front end of the C oracle core (pcast_oracle.c).

Test infrastructure: only the tests, the smoke check and the CPU-baseline leg
of the benchmark use this package.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pcast_oracle.c")
_LIB = os.path.join(_HERE, "_pcast_oracle.so")
_lock = threading.Lock()
_lib = None

MODE_IDS = {"kernel": 0, "pages": 1, "bf16": 2, "nocast": 3}
# Relative perturbation of S*p within which a rounding decision counts as a
# near tie (bounds the fp32 error of the GPU's logits and exp2 many times over).
DEFAULT_EPS = 2.0 ** -12


def build() -> str:
    """Compile pcast_oracle.c into _pcast_oracle.so (always recompiles)."""
    tmp = _LIB + ".tmp"
    subprocess.run(["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC",
                    "-shared", _SRC, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB):
                build()
            lib = ctypes.CDLL(_LIB)
            P = ctypes.c_void_p
            lib.oracle_rows.argtypes = [P, P, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_int, P,
                                        ctypes.c_int64, ctypes.c_double, P, P, P, P, ctypes.c_int]
            lib.oracle_rows.restype = ctypes.c_int
            for name in ("oracle_e4m3_rne_n", "oracle_bf16_rne_n"):
                fn = getattr(lib, name)
                fn.argtypes = [P, P, ctypes.c_int64]
                fn.restype = None
            lib.oracle_max_threads.restype = ctypes.c_int
            _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def e4m3_rne(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty_like(x)
    _load().oracle_e4m3_rne_n(x.ctypes.data, y.ctypes.data, x.size)
    return y


def bf16_rne(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty_like(x)
    _load().oracle_bf16_rne_n(x.ctypes.data, y.ctypes.data, x.size)
    return y


def _ptr(a):
    return None if a is None else a.ctypes.data


def rows(q_bits, k_bits, v_bits, bias, causal: bool, S: float, order: int, mode: str = "kernel",
         row_ids=None, bc: int = 64, eps: float = DEFAULT_EPS, want_exact: bool = True,
         nthreads: int = 0):
    """Run the oracle on the listed rows of bf16 inputs [B,Hq,N,d] / [B,Hkv,N,d].

    row_ids: flat ids (b*Hq + h)*N + i, or None for every row.  Returns a dict
    with o2 [R,d], o1 [R,d] (if want_exact), slack [R] and the counters
    total / zero / zero_amb / zero_beyond_block0 [R].
    """
    q = np.ascontiguousarray(q_bits, dtype=np.uint16)
    k = np.ascontiguousarray(k_bits, dtype=np.uint16)
    v = np.ascontiguousarray(v_bits, dtype=np.uint16)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    assert k.shape == (B, Hkv, N, d) and v.shape == k.shape
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    assert b is None or b.shape == (N,)
    ids = None if row_ids is None else np.ascontiguousarray(row_ids, dtype=np.int64)
    R = B * Hq * N if ids is None else ids.size
    o2 = np.empty((R, d))
    o1 = np.empty((R, d)) if want_exact else None
    slack = np.empty(R)
    cnt = np.empty((R, 4), dtype=np.int64)
    nt = nthreads if nthreads > 0 else (os.cpu_count() or 1)
    rc = _load().oracle_rows(q.ctypes.data, k.ctypes.data, v.ctypes.data, _ptr(b), B, Hq, Hkv, N,
                             d, int(bool(causal)), float(S), int(order), MODE_IDS[mode], bc,
                             _ptr(ids), R, float(eps), o2.ctypes.data, _ptr(o1),
                             slack.ctypes.data, cnt.ctypes.data, nt)
    if rc != 0:
        raise ValueError("oracle_rows rejected its arguments")
    out = {"o2": o2, "slack": slack, "total": cnt[:, 0], "zero": cnt[:, 1],
           "zero_amb": cnt[:, 2], "zero_beyond_block0": cnt[:, 3]}
    if want_exact:
        out["o1"] = o1
    return out

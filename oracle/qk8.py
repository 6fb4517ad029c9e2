"""FP8 logits, an extension of the P-cast path: Q and K rounded to E4M3 with a
per-head power-of-two scale before Q K^T.

TEST INFRASTRUCTURE: only the tests, the smoke check and the CPU-baseline leg of
the benchmark use this package.

The FlashAttention blog ("FA3: Meccanica della tramoggia") names FP8 inputs
with a per-block descale as the way to the FP8 matrix rate; the P-cast summaries
only cast P.  Reading taken here (the plainest one that keeps every step exact):

* the scale of a head is the smallest power of two 2^e with max|x| <= 448 * 2^e,
  so x / 2^e is exact in fp32 and no value saturates; a head of zeros takes e = 0;
* a value enters the logits as E4M3_RNE(x / 2^e) * 2^e.  With 3 mantissa bits and
  an exponent well inside bf16's range that product is exactly a bf16 value, so
  the rest of the oracle runs unchanged on the quantised Q and K.
"""
from __future__ import annotations

import math

import numpy as np

from .e4m3 import E4M3_MAX, e4m3_rne


def head_scale_exp(amax: float) -> int:
    """Smallest integer e with amax <= 448 * 2^e (0 for amax == 0)."""
    amax = float(amax)
    if amax == 0.0:
        return 0
    m, E = math.frexp(amax)  # amax = m * 2^E, m in [0.5, 1); 448 = 0.875 * 2^9
    return E - 9 if m <= 0.875 else E - 8


def _bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    u = (np.asarray(bits).astype(np.uint32) & 0xFFFF) << 16
    return u.view(np.float32).astype(np.float64)


def _f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """bf16 bits of values that are exactly representable in bf16 (checked)."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("value not representable in bf16")
    return (u >> 16).astype(np.uint16)


def quantize_heads(bits: np.ndarray):
    """Quantise a bf16 tensor [B, H, N, d] head by head.

    Returns (bf16 bits of E4M3_RNE(x / 2^e) * 2^e, exponents e [B, H]).
    """
    x = _bf16_bits_to_f64(bits)
    B, H = x.shape[:2]
    exps = np.zeros((B, H), dtype=np.int64)
    out = np.empty_like(x)
    for b in range(B):
        for h in range(H):
            e = head_scale_exp(np.max(np.abs(x[b, h])))
            exps[b, h] = e
            q = e4m3_rne(np.ldexp(x[b, h], -e))
            assert np.max(np.abs(q)) <= E4M3_MAX
            out[b, h] = np.ldexp(q, e)
    return _f64_to_bf16_bits(out).reshape(np.shape(bits)), exps

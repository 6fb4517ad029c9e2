"""FP8 logits, an extension of the P-cast path: Q and K rounded to E4M3 with
power-of-two block scales before Q K^T.

TEST INFRASTRUCTURE: only the tests, the smoke check and the CPU-baseline leg of
the benchmark use this package.

The FlashAttention blog ("FA3: Meccanica della tramoggia", item 3) describes
FP8 attention inputs quantised block by block, one scale per block; the P-cast
summaries only cast P.  Reading taken here (the plainest one that keeps every
step exact):

* blocks: every query row is a block of Q (the finest block of rows), and every
  64-key block of a head is a block of K (the key block of the online softmax);
* the scale of a block is the smallest power of two 2^e with
  max|x| <= 448 * 2^e over the block, so x / 2^e is exact and no value
  saturates; a block of zeros takes e = 0;
* a value enters the logits as E4M3_RNE(x / 2^e) * 2^e.  With 3 mantissa bits
  and an exponent well inside bf16's range that product is exactly a bf16
  value, so the rest of the oracle runs unchanged on the quantised Q and K, and
  the logit of (i, j) is sum_d code_q * code_k * 2^(e_i + e_block(j)) / sqrt(d).
"""
from __future__ import annotations

import math

import numpy as np

from .e4m3 import E4M3_MAX, e4m3_rne

Q_BLOCK_ROWS = 1    # one scale per query row
K_BLOCK_ROWS = 64   # one scale per key block


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


def scale_exps(amax) -> np.ndarray:
    """head_scale_exp applied elementwise to an array of maxima."""
    a = np.asarray(amax, dtype=np.float64)
    m, E = np.frexp(a)
    e = np.where(m <= 0.875, E - 9, E - 8)
    return np.where(a == 0.0, 0, e).astype(np.int64)


def quantize_blocks(bits: np.ndarray, rows: int):
    """Quantise a bf16 tensor [B, H, N, d] in blocks of `rows` consecutive rows
    of one head; a partial last block (N % rows != 0) holds the rows that exist,
    so its scale is that of their max.

    Returns (bf16 bits of E4M3_RNE(x / 2^e) * 2^e, exponents e [B, H, ceil(N / rows)]).
    """
    x = _bf16_bits_to_f64(bits)
    B, H, N, d = x.shape
    nb = -(-N // rows)
    xp = np.zeros((B, H, nb * rows, d))  # rows past N are zeros: they leave every block max unchanged
    xp[:, :, :N] = x
    blocks = xp.reshape(B, H, nb, rows * d)
    exps = scale_exps(np.max(np.abs(blocks), axis=3))
    e = exps[..., None]
    q = e4m3_rne(np.ldexp(blocks, -e))
    assert q.size == 0 or np.max(np.abs(q)) <= E4M3_MAX
    out = np.ldexp(q, e).reshape(xp.shape)[:, :, :N]
    return _f64_to_bf16_bits(out).reshape(np.shape(bits)), exps


def quantize_q(bits: np.ndarray):
    """Q with one scale per row: (dequantised bf16 bits, exponents [B, H, N])."""
    return quantize_blocks(bits, Q_BLOCK_ROWS)


def quantize_k(bits: np.ndarray):
    """K with one scale per 64-key block: (dequantised bf16 bits, exponents [B, H, ceil(N/64)])."""
    return quantize_blocks(bits, K_BLOCK_ROWS)


# ---------------------------------------------------------------------------
# Random rotation before the quantisation ("FP8 con elaborazione incoerente" in the
# FlashAttention blog's FA3 section: Q and K are rotated by a random orthogonal
# matrix so that an outlier's magnitude spreads over all coordinates).  Reading:
# the randomised Hadamard transform x -> x diag(sigma) H with H the d x d Sylvester
# matrix of +-1 and sigma random signs (an input).  It is not normalised: since
# H H^T = d I, (q diag(sigma) H) . (k diag(sigma) H) = d (q . k), and the factor d
# (a power of two) is taken out of K exactly.  In fp64 the rotation of bf16 inputs
# is exact.
# ---------------------------------------------------------------------------
def hadamard(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order d (a power of two), entries +-1."""
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    if h.shape[0] != d:
        raise ValueError("d must be a power of two")
    return h


def rotate(bits: np.ndarray, signs) -> np.ndarray:
    """x diag(signs) H for every row of a bf16 tensor [..., d], fp64."""
    x = _bf16_bits_to_f64(bits)
    d = x.shape[-1]
    return (x * np.asarray(signs, dtype=np.float64)) @ hadamard(d)


def quantize_values(x: np.ndarray, rows: int):
    """quantize_blocks on fp64 values [B, H, N, d]: (E4M3_RNE(x / 2^e) * 2^e, e); a
    partial last block holds the rows that exist."""
    B, H, N, d = x.shape
    nb = -(-N // rows)
    xp = np.zeros((B, H, nb * rows, d))  # rows past N are zeros: they leave every block max unchanged
    xp[:, :, :N] = x
    blocks = xp.reshape(B, H, nb, rows * d)
    exps = scale_exps(np.max(np.abs(blocks), axis=3))
    q = e4m3_rne(np.ldexp(blocks, -exps[..., None]))
    assert q.size == 0 or np.max(np.abs(q)) <= E4M3_MAX
    return np.ldexp(q, exps[..., None]).reshape(xp.shape)[:, :, :N], exps


def quantize_rotated(q_bits: np.ndarray, k_bits: np.ndarray, signs):
    """Rotated, then quantised Q (per row) and K (per 64-key block), as bf16 bits whose
    plain dot products are those of the original logits' inputs: Q~ and K~ / d.
    Returns (q bits, k bits, q exps [B, H, N], k exps [B, Hkv, ceil(N/64)])."""
    d = np.shape(q_bits)[-1]
    qv, eq = quantize_values(rotate(q_bits, signs), Q_BLOCK_ROWS)
    kv, ek = quantize_values(rotate(k_bits, signs), K_BLOCK_ROWS)
    return _f64_to_bf16_bits(qv), _f64_to_bf16_bits(kv / d), eq, ek

"""Software FP8 E4M3 (OCP "e4m3fn") and bf16 rounding, in fp64.

Test infrastructure: only the tests, the smoke check and the CPU-baseline leg
of the benchmark use this package.

Format (the one the P-cast pages describe: 3 mantissa bits, largest finite
value 448, smallest normal 2^-6, values at or below 2^-10 round to zero --
P-cast summary, sections "Metodologia e Analisi" and "Ottimizzazione 2"):

* code = s eeee mmm, exponent bias 7
* e = 0:       value = m * 2^-9            (subnormal; m = 0 is +/-0)
* e = 1..15:   value = (1 + m/8) * 2^(e-7)  except s.1111.111 = NaN
* no infinities; 448 = 0x7E is the largest finite value.

Encoding is round-to-nearest, ties-to-even onto that grid, with magnitudes
above 448 saturating to 448 (the kernel clamps before converting).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E4M3_MIN_NORMAL = 2.0 ** -6
E4M3_MIN_SUBNORMAL = 2.0 ** -9
E4M3_ZERO_THRESHOLD = 2.0 ** -10  # largest magnitude that encodes to 0


def decode_code(code: int) -> float:
    """Value of one 8-bit code, straight from the field definition."""
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        mag = m * 2.0 ** -9
    else:
        mag = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


DECODE_TABLE = np.array([decode_code(c) for c in range(256)], dtype=np.float64)


def grid() -> np.ndarray:
    """The 127 distinct non-negative finite E4M3 values, ascending."""
    v = DECODE_TABLE[:128]
    return np.unique(v[np.isfinite(v)])


def e4m3_rne(x) -> np.ndarray:
    """Round fp64 values onto the E4M3 grid (RNE, saturating at +/-448).

    Within a binade [2^E, 2^(E+1)) with E >= -6 the grid step is 2^(E-3);
    below 2^-6 it is the subnormal step 2^-9.  Dividing by a power of two is
    exact, so ``rint(|x| / step) * step`` is the exact RNE result.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, e = np.frexp(a)                    # a = f * 2^e, f in [0.5, 1)
    binade = e.astype(np.int64) - 1       # a in [2^binade, 2^(binade+1))
    step_exp = np.where(a < E4M3_MIN_NORMAL, -9, binade - 3)
    step = np.ldexp(1.0, step_exp)
    q = np.rint(a / step) * step          # np.rint rounds half to even
    q = np.minimum(q, E4M3_MAX)
    q = np.where(np.isnan(x), np.nan, q)
    return np.copysign(q, x)


def e4m3_encode(x) -> np.ndarray:
    """uint8 codes of ``e4m3_rne(x)`` (NaN -> 0x7F)."""
    v = e4m3_rne(x)
    pos = DECODE_TABLE[:127]                       # codes 0x00..0x7E, ascending values
    idx = np.searchsorted(pos, np.abs(v))
    idx = np.clip(idx, 0, 126)
    codes = idx.astype(np.uint8) | np.where(np.signbit(v), 0x80, 0).astype(np.uint8)
    return np.where(np.isnan(v), np.uint8(0x7F), codes).astype(np.uint8)


def bf16_rne(x) -> np.ndarray:
    """Round fp64 values to bfloat16 (8 significant bits), RNE, no overflow handling."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, e = np.frexp(a)
    step_exp = np.maximum(e.astype(np.int64) - 8, -133)   # bf16 subnormal step 2^-133
    step = np.ldexp(1.0, step_exp)
    return np.copysign(np.rint(a / step) * step, x)


def quant_step_max(S: float) -> float:
    """d_p(S): the largest grid spacing met by values in (0, S], divided by S.

    This is the maximum normalised quantisation step of the P-cast summary
    (section "Ottimizzazione 2", point 2), computed by brute force from the
    grid.  Defined for 0 < S <= 448.
    """
    g = grid()
    lo, hi = g[:-1], g[1:]
    mask = lo < S
    return float(np.max((hi - lo)[mask]) / S)

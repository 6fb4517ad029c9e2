"""Per-row diagnostics of the P-cast pipeline: log-sum-exp and lost non-sink mass.

TEST INFRASTRUCTURE: only the tests, the smoke check and the CPU-baseline leg of
the benchmark use this module.

Definitions (P-cast summary, sections 1 and 2: the cast silently zeroes part of
the non-sink probability mass; "30-40 % of the non-sink mass" in the Chinese
page's popular section):

* s_ij = q_i . k_j / sqrt(d) + bias_j over the visible keys j of row i;
  lse_i = ln sum_j exp(s_ij);
* the weight of key j is its exact softmax weight w_ij = exp(s_ij - m_i), m_i the
  row max; its E4M3 code is the pipeline's, E4M3(S * exp(s_ij - M_i(j))), M_i(j)
  the running max just after visiting the block of key j in the given order (the
  telescoped form of the block recurrence);
* lost_i = sum_{j non-sink, code 0} w_ij / sum_{j non-sink} w_ij (0 if the row has
  no non-sink key).  A key is a sink when its bias is non-zero.

Also returned per row: the number of non-sink codes at zero (the same count as the
oracle's underflow counter) and lost_amb_i, the share of non-sink mass whose zero /
non-zero decision lies within a relative eps of the threshold 2^-10, for tolerances.
"""
from __future__ import annotations

import math

import numpy as np

from .e4m3 import E4M3_ZERO_THRESHOLD, e4m3_rne


def _bf16(bits):
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _row_logits(q_rows, pos, k, bias, causal):
    s = (q_rows @ k.T) / math.sqrt(q_rows.shape[1])
    if bias is not None:
        s = s + np.asarray(bias, dtype=np.float64)[None, :]
    if causal:
        s = np.where(np.arange(k.shape[0])[None, :] <= pos[:, None], s, -np.inf)
    return s


def _running_max(s, order, bc):
    R, N = s.shape
    nblk = -(-N // bc)  # a partial last block holds the keys from its start up to N
    sp = np.pad(s, ((0, 0), (0, nblk * bc - N)), constant_values=-np.inf)
    bmax = sp.reshape(R, nblk, bc).max(axis=2)
    if order == 0:
        run = np.maximum.accumulate(bmax, axis=1)
    else:
        run = np.maximum.accumulate(bmax[:, ::-1], axis=1)[:, ::-1]
    return np.repeat(run, bc, axis=1)[:, :N]


def rows(q_bits, k_bits, bias, causal: bool, S: float, order: int, row_ids=None, bc: int = 64,
         eps: float = 2.0 ** -14):
    """Diagnostics for the listed rows (flat ids (b*Hq + h)*N + i; all rows if None).

    Returns a dict of [R] arrays: lse, lost, lost_amb, zero (int).
    """
    B, Hq, N, d = q_bits.shape
    Hkv = k_bits.shape[1]
    ids = np.arange(B * Hq * N) if row_ids is None else np.asarray(row_ids, dtype=np.int64)
    nonsink = np.ones(N, dtype=bool) if bias is None else (np.asarray(bias) == 0)
    out = {k: np.zeros(ids.size) for k in ("lse", "lost", "lost_amb")}
    out["zero"] = np.zeros(ids.size, dtype=np.int64)
    bh = ids // N
    for key in np.unique(bh):
        sel = np.nonzero(bh == key)[0]
        b, h = divmod(int(key), Hq)
        pos = ids[sel] % N
        q = _bf16(q_bits[b, h][pos])
        k = _bf16(k_bits[b, h // (Hq // Hkv)])
        s = _row_logits(q, pos, k, bias, causal)
        vis = np.isfinite(s)
        m = np.max(s, axis=1, keepdims=True)
        with np.errstate(invalid="ignore"):
            w = np.where(vis, np.exp(s - m), 0.0)
            Mj = _running_max(s, order, bc)
            sp = np.where(vis, S * np.exp(s - Mj), np.inf)     # S * p of each visible key
        zero = vis & (e4m3_rne(np.where(vis, sp, 0.0)) == 0.0)
        amb = vis & (np.abs(sp - E4M3_ZERO_THRESHOLD) <= eps * E4M3_ZERO_THRESHOLD)
        ns = vis & nonsink[None, :]
        tot = np.sum(np.where(ns, w, 0.0), axis=1)
        safe = np.where(tot > 0, tot, 1.0)
        out["lse"][sel] = m[:, 0] + np.log(np.sum(w, axis=1))
        out["lost"][sel] = np.where(tot > 0, np.sum(np.where(ns & zero, w, 0.0), axis=1) / safe, 0.0)
        out["lost_amb"][sel] = np.where(tot > 0, np.sum(np.where(ns & amb, w, 0.0), axis=1) / safe, 0.0)
        out["zero"][sel] = np.sum(ns & zero, axis=1)
    return out

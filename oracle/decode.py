"""Decode with split KV: a few query rows at the end of a sequence, the keys cut
into contiguous ranges that each run the P-cast block pipeline on their own, and
the ranges' results merged.

TEST INFRASTRUCTURE: only the tests, the smoke check and the CPU-baseline leg of
the benchmark use this module.

Reading (the FlashAttention blog, "La ricorrenza softmax online": the running
statistics (m, l, A) of two key sets combine by rescaling both to the larger max;
P-cast summary, sections 1 and 2: the cast is taken relative to the running max
that the pipeline holds when the block is visited):

* Q rows [B][Hq][Nq][d] sit at the last Nq positions of a sequence of Nk keys:
  row i is at position Nk - Nq + i and sees keys j <= Nk - Nq + i (causal,
  bottom-right aligned); every key is visible when Nq = 1;
* the keys are cut into ranges of `split_keys` keys (a multiple of 64): range r
  holds keys [r split_keys, (r+1) split_keys);
* each range runs the pipeline of the P-cast path over its own 64-key blocks,
  forward or reverse within the range, from m = -inf, l = 0, A = 0:
  m' = max(m, block max), alpha = e^(m - m'), p = e^(s - m'), l = alpha l + sum p,
  c = E4M3(S p), A = alpha A + sum c vhat (vhat = E4M3(V) in kernel mode);
* merge: M = max_r m_r, O = sum_r e^(m_r - M) A_r / (S sum_r e^(m_r - M) l_r).

One range (split_keys >= Nk) is the P-cast path itself on that row.  Counters per
row: non-sink visible keys, and those whose code is 0.
"""
from __future__ import annotations

import math

import numpy as np

from .e4m3 import E4M3_ZERO_THRESHOLD, e4m3_rne


def _bf16(bits):
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _cast(x, mode):
    if mode == "kernel":
        return e4m3_rne(x)
    if mode == "nocast":
        return x
    raise ValueError(mode)


def _near(x, eps, mode):
    """(near-tie flag, size of the code step there) for each S*p value."""
    lo, hi = _cast(x * (1.0 - eps), mode), _cast(x * (1.0 + eps), mode)
    return lo != hi, hi - lo


def rows(q_bits, k_bits, v_bits, bias, S: float, order: int, split_keys: int, mode: str = "kernel",
         bc: int = 64, eps: float = 2.0 ** -14):
    """O2, O1, slack and counters for every decode row.

    q_bits [B,Hq,Nq,d], k_bits and v_bits [B,Hkv,Nk,d] (bf16 bits), bias [Nk] or None.
    Returns a dict: o2, o1 [B,Hq,Nq,d]; slack, total, zero, zero_amb [B,Hq,Nq].
    """
    B, Hq, Nq, d = q_bits.shape
    Hkv, Nk = k_bits.shape[1], k_bits.shape[2]
    if split_keys % bc:
        raise ValueError("split_keys must be a multiple of the block size")
    G = Hq // Hkv
    nonsink = np.ones(Nk, dtype=bool) if bias is None else (np.asarray(bias) == 0)
    bvec = np.zeros(Nk) if bias is None else np.asarray(bias, dtype=np.float64)
    o2 = np.zeros((B, Hq, Nq, d))
    o1 = np.zeros((B, Hq, Nq, d))
    slack = np.zeros((B, Hq, Nq))
    total = np.zeros((B, Hq, Nq), dtype=np.int64)
    zero = np.zeros((B, Hq, Nq), dtype=np.int64)
    zero_amb = np.zeros((B, Hq, Nq), dtype=np.int64)
    for b in range(B):
        for hk in range(Hkv):
            k = _bf16(k_bits[b, hk])
            v = _bf16(v_bits[b, hk])
            vh = e4m3_rne(v) if mode == "kernel" else v
            vmax = np.max(np.abs(vh), axis=1)
            for h in range(hk * G, (hk + 1) * G):
                for i in range(Nq):
                    pos = Nk - Nq + i
                    q = _bf16(q_bits[b, h, i])
                    s = k[:pos + 1] @ q / math.sqrt(d) + bvec[:pos + 1]
                    n = pos + 1
                    # exact attention
                    w = np.exp(s - s.max())
                    o1[b, h, i] = w @ v[:n] / w.sum()
                    # each range on its own
                    parts = []
                    for r0 in range(0, n, split_keys):
                        r1 = min(r0 + split_keys, n)
                        blocks = list(range(r0, r1, bc))
                        if order:
                            blocks = blocks[::-1]
                        m, l, A = -np.inf, 0.0, np.zeros(d)
                        Mj = np.zeros(r1 - r0)              # running max when each key's block is visited
                        for t0 in blocks:
                            js = np.arange(t0, min(t0 + bc, r1))
                            mp = max(m, float(np.max(s[js])))
                            a = 0.0 if m == -np.inf else math.exp(m - mp)
                            p = np.exp(s[js] - mp)
                            l = a * l + float(np.sum(p))
                            c = _cast(S * p, mode)
                            A = a * A + c @ vh[js]
                            m = mp
                            Mj[js - r0] = mp
                        parts.append((m, l, A, r0, r1, Mj))
                    M = max(pp[0] for pp in parts)
                    L = sum(math.exp(pp[0] - M) * pp[1] for pp in parts)
                    o2[b, h, i] = sum(math.exp(pp[0] - M) * pp[2] for pp in parts) / (S * L)
                    # counters and slack, key by key
                    for m_r, _, _, r0, r1, Mj in parts:
                        js = np.arange(r0, r1)
                        sp = S * np.exp(s[js] - Mj)
                        c = _cast(sp, mode)
                        near, step = _near(sp, eps, mode)
                        ns = nonsink[js]
                        total[b, h, i] += int(ns.sum())
                        zero[b, h, i] += int(np.sum(ns & (c == 0)))
                        zamb = np.abs(sp - E4M3_ZERO_THRESHOLD) <= eps * E4M3_ZERO_THRESHOLD
                        zero_amb[b, h, i] += int(np.sum(ns & zamb))
                        slack[b, h, i] += float(np.sum(np.where(near, step * np.exp(Mj - M) * vmax[js], 0.0))) / (S * L)
    return {"o2": o2, "o1": o1, "slack": slack, "total": total, "zero": zero, "zero_amb": zero_amb}

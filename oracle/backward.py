"""Backward of the attention forward by recomputation from the log-sum-exp.

TEST INFRASTRUCTURE: only the tests, the smoke check and the CPU-baseline leg of
the benchmark use this module.

The FlashAttention blog ("Passaggio all'indietro: ricalcolo anziché archiviazione")
keeps only O and the softmax statistics of the forward and recomputes the
probability tiles from Q, K in the backward.  Reading taken here for the P-cast
path: the cast is passed straight through (its derivative taken as 1), so with
s_ij = q_i . k_j / sqrt(d) + bias_j over the visible keys and lse_i the row's
log-sum-exp,

    P_ij = exp(s_ij - lse_i)            dV_j = sum_i P_ij dO_i
    dP_ij = dO_i . v_j                  D_i  = dO_i . O_i   (O: the forward's output)
    dS_ij = P_ij (dP_ij - D_i)          dQ_i = sum_j dS_ij k_j / sqrt(d)
                                        dK_j = sum_i dS_ij q_i / sqrt(d)

with dK and dV of a kv head summed over the query heads that read it.  With O and
lse of exact attention these are the exact gradients of softmax(Q K^T/sqrt(d) + b) V.
"""
from __future__ import annotations

import math

import numpy as np


def _bf16(bits):
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def grads(q_bits, k_bits, v_bits, o, do_bits, lse, bias, causal: bool, with_bounds: bool = False):
    """fp64 dQ [B,Hq,N,d], dK and dV [B,Hkv,N,d] from bf16 Q, K, V, dO, the forward's O and
    lse [B,Hq,N].  with_bounds: also return the magnitude sums |dS||K|/sqrt(d), |dS|^T|Q|/sqrt(d)
    and |P|^T|dO| that bound the rounding of dS and P to bf16 ("dq", "dk", "dv"), and
    P (A + E) |K| / sqrt(d), (P (A + E))^T |Q| / sqrt(d) with A_ij = |dO_i| . |v_j| and
    E_i = |dO_i| . |O_i|, which bound the effect of an error in dP - D relative to the
    magnitudes it is summed from ("dq2", "dk2")."""
    q, k, v, do = _bf16(q_bits), _bf16(k_bits), _bf16(v_bits), _bf16(do_bits)
    o = np.asarray(o, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    sc = 1.0 / math.sqrt(d)
    bvec = np.zeros(N) if bias is None else np.asarray(bias, dtype=np.float64)
    dq = np.zeros_like(q)
    dk = np.zeros((B, Hkv, N, d))
    dv = np.zeros((B, Hkv, N, d))
    bnd = {"dq": np.zeros_like(q), "dk": np.zeros((B, Hkv, N, d)), "dv": np.zeros((B, Hkv, N, d)),
           "dq2": np.zeros_like(q), "dk2": np.zeros((B, Hkv, N, d))}
    mask = np.tril(np.ones((N, N), dtype=bool)) if causal else np.ones((N, N), dtype=bool)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            s = q[b, h] @ k[b, g].T * sc + bvec[None, :]
            p = np.where(mask, np.exp(np.where(mask, s, 0.0) - lse[b, h][:, None]), 0.0)
            dp = do[b, h] @ v[b, g].T
            D = np.sum(do[b, h] * o[b, h], axis=1)
            ds = p * (dp - D[:, None])
            dv[b, g] += p.T @ do[b, h]
            dq[b, h] = ds @ k[b, g] * sc
            dk[b, g] += ds.T @ q[b, h] * sc
            if with_bounds:
                bnd["dq"][b, h] = np.abs(ds) @ np.abs(k[b, g]) * sc
                bnd["dk"][b, g] += np.abs(ds).T @ np.abs(q[b, h]) * sc
                bnd["dv"][b, g] += np.abs(p).T @ np.abs(do[b, h])
                pe = p * (np.abs(do[b, h]) @ np.abs(v[b, g]).T + np.sum(np.abs(do[b, h] * o[b, h]), axis=1)[:, None])
                bnd["dq2"][b, h] = pe @ np.abs(k[b, g]) * sc
                bnd["dk2"][b, g] += pe.T @ np.abs(q[b, h]) * sc
    if with_bounds:
        return dq, dk, dv, bnd
    return dq, dk, dv


def forward_exact(q_bits, k_bits, v_bits, bias, causal: bool):
    """Exact attention O [B,Hq,N,d] and lse [B,Hq,N] in fp64 (for pins and inputs)."""
    q, k, v = _bf16(q_bits), _bf16(k_bits), _bf16(v_bits)
    B, Hq, N, d = q.shape
    G = Hq // k.shape[1]
    bvec = np.zeros(N) if bias is None else np.asarray(bias, dtype=np.float64)
    o = np.zeros_like(q)
    lse = np.zeros((B, Hq, N))
    for b in range(B):
        for h in range(Hq):
            s = q[b, h] @ k[b, h // G].T / math.sqrt(d) + bvec[None, :]
            if causal:
                s = np.where(np.tril(np.ones((N, N), dtype=bool)), s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            w = np.exp(s - m)
            lse[b, h] = m[:, 0] + np.log(w.sum(axis=1))
            o[b, h] = (w / w.sum(axis=1, keepdims=True)) @ v[b, h // G]
    return o, lse


def grads_sampled(q_bits, k_bits, v_bits, o, do_bits, lse, bias, causal: bool, rows, keys):
    """The same gradients one by one: dQ of the listed rows (b, h, i) and dK, dV of the
    listed keys (b, kv head, j), each from its own row or column of the formulas, with
    the bf16-rounding magnitude sums as in grads().  Returns (dq [R,d], dk [K,d],
    dv [K,d], bounds dict)."""
    B, Hq, N, d = np.shape(q_bits)
    Hkv = np.shape(k_bits)[1]
    G = Hq // Hkv
    sc = 1.0 / math.sqrt(d)
    bvec = np.zeros(N) if bias is None else np.asarray(bias, dtype=np.float64)
    o = np.asarray(o)
    lse = np.asarray(lse)
    out_q, bq, bq2 = [], [], []
    for b, h, i in rows:
        g = h // G
        qi, k, v = _bf16(q_bits[b, h, i]), _bf16(k_bits[b, g]), _bf16(v_bits[b, g])
        do_i = _bf16(do_bits[b, h, i])
        n = i + 1 if causal else N
        s = k[:n] @ qi * sc + bvec[:n]
        p = np.exp(s - float(lse[b, h, i]))
        ds = p * (v[:n] @ do_i - float(np.dot(do_i, o[b, h, i].astype(np.float64))))
        out_q.append(ds @ k[:n] * sc)
        bq.append(np.abs(ds) @ np.abs(k[:n]) * sc)
        pe = p * (np.abs(v[:n]) @ np.abs(do_i) + float(np.sum(np.abs(do_i * o[b, h, i].astype(np.float64)))))
        bq2.append(pe @ np.abs(k[:n]) * sc)
    out_k, out_v, bk, bv, bk2 = [], [], [], [], []
    for b, g, j in keys:
        kj, vj = _bf16(k_bits[b, g, j]), _bf16(v_bits[b, g, j])
        dk, dv = np.zeros(d), np.zeros(d)
        ak, av, ak2 = np.zeros(d), np.zeros(d), np.zeros(d)
        for h in range(g * G, (g + 1) * G):
            i0 = j if causal else 0
            qh, doh = _bf16(q_bits[b, h, i0:]), _bf16(do_bits[b, h, i0:])
            oh = o[b, h, i0:].astype(np.float64)
            s = qh @ kj * sc + bvec[j]
            p = np.exp(s - lse[b, h, i0:].astype(np.float64))
            ds = p * (doh @ vj - np.sum(doh * oh, axis=1))
            dk += ds @ qh * sc
            dv += p @ doh
            ak += np.abs(ds) @ np.abs(qh) * sc
            av += np.abs(p) @ np.abs(doh)
            pe = p * (np.abs(doh) @ np.abs(vj) + np.sum(np.abs(doh * oh), axis=1))
            ak2 += pe @ np.abs(qh) * sc
        out_k.append(dk)
        out_v.append(dv)
        bk.append(ak)
        bv.append(av)
        bk2.append(ak2)
    return (np.array(out_q), np.array(out_k), np.array(out_v),
            {"dq": np.array(bq), "dk": np.array(bk), "dv": np.array(bv), "dq2": np.array(bq2),
             "dk2": np.array(bk2)})

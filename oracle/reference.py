"""NumPy fp64 oracle for P-cast attention (small sizes; the C core scales it up).

Test infrastructure: only the tests, the smoke check and the CPU-baseline leg
of the benchmark use this package.  It shares no code with the HIP path.

Two results are defined here.

O1 -- exact attention (FlashAttention blog, section "Perché l'attenzione è
legata alla memoria": O = softmax(Q K^T / sqrt(d)) V), with the per-key
additive bias of the sink setting and a square causal mask (key j visible to
query i iff j <= i, the blog's causal-masking section).  Computed in fp64 on
the exact bf16 input values.

O2 -- the P-cast block pipeline.  The online-softmax recurrence of the blog's
"L'algoritmo Flash Attention" and "La ricorrenza softmax online" sections, in
the running-max form in which the probability tile is taken relative to the
running maximum that includes the current block (the form in which the sink
"inflates the running max", P-cast summary section 1), with the deferred
normalisation of the blog's FA2 section, and with the P-cast of the P-cast
summary (P multiplied by a static S, cast to E4M3 before P.V, divided by S in
the epilogue).  Keys are visited in blocks of ``bc``; order 0 visits blocks
0 -> last, order 1 visits last -> 0 (P-cast summary, "Ottimizzazione 1").

Per row, with running max m = -inf, running sum l = 0, accumulator A = 0:
    for each visited block J (keys of the block that the row may see):
        m'  = max(m, max_J s_j)
        a   = exp(m - m')            (0 while m = -inf)
        p_j = exp(s_j - m')          for j in J
        l   = a l + sum_J p_j        (un-cast p)
        c_j = cast(S p_j)
        A   = a A + sum_J c_j vhat_j
        m   = m'
    O2 = A / (S l)

Modes (what ``cast`` and ``vhat`` are):
    "kernel": c = E4M3(S p), vhat = E4M3(V)   -- what an FP8 x FP8 MFMA sees
    "pages":  c = E4M3(S p), vhat = V         -- Q, K, V kept exact, only P cast
                                                 (the summary's kernel-faithful
                                                 simulation, section 2, point 4)
    "bf16":   c = bf16(p),   vhat = V, S := 1 -- the no-P-cast bf16 path
    "nocast": c = S p,       vhat = V         -- exact; must equal O1

Counters per row (non-sink = bias_j == 0, or every key when there is no bias):
total = non-sink pairs the row evaluates, zero = those whose code is 0.
"""
from __future__ import annotations

import math

import numpy as np

from .e4m3 import bf16_rne, e4m3_rne

MODES = ("kernel", "pages", "bf16", "nocast")


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns as fp64."""
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def logits(q: np.ndarray, k: np.ndarray, bias, causal: bool) -> np.ndarray:
    """s = q k^T / sqrt(d) + bias for one head, -inf where the causal mask hides a key.

    q: [Nq, d] fp64 rows at positions 0..Nq-1; k: [N, d] fp64.
    """
    d = q.shape[1]
    s = (q @ k.T) / math.sqrt(d)
    if bias is not None:
        s = s + np.asarray(bias, dtype=np.float64)[None, :]
    if causal:
        i = np.arange(q.shape[0])[:, None]
        j = np.arange(k.shape[0])[None, :]
        s = np.where(j <= i, s, -np.inf)
    return s


def exact_attention(s: np.ndarray, v: np.ndarray) -> np.ndarray:
    """O1 = softmax(s) v, two-pass, fp64."""
    m = np.max(s, axis=1, keepdims=True)
    w = np.exp(s - m)
    return (w @ v) / np.sum(w, axis=1, keepdims=True)


def _cast(y: np.ndarray, mode: str) -> np.ndarray:
    if mode in ("kernel", "pages"):
        return e4m3_rne(y)
    if mode == "bf16":
        return bf16_rne(y)
    if mode == "nocast":
        return y
    raise ValueError(mode)


def _vhat(v: np.ndarray, mode: str) -> np.ndarray:
    return e4m3_rne(v) if mode == "kernel" else v


def _scale(S: float, mode: str) -> float:
    return 1.0 if mode == "bf16" else float(S)


def emulate_sequential(s: np.ndarray, v: np.ndarray, S: float, order: int, mode: str,
                       bc: int = 64, nonsink=None):
    """O2 row by row and block by block, exactly as the recurrence reads.

    s: [R, N] logits (-inf = masked); v: [N, d].  Returns (O2 [R, d],
    total [R], zero [R]).
    """
    S = _scale(S, mode)
    vh = _vhat(v, mode)
    R, N = s.shape
    nonsink = np.ones(N, dtype=bool) if nonsink is None else np.asarray(nonsink, dtype=bool)
    out = np.zeros((R, v.shape[1]))
    total = np.zeros(R, dtype=np.int64)
    zero = np.zeros(R, dtype=np.int64)
    nblk = (N + bc - 1) // bc
    for r in range(R):
        m, l, A = -np.inf, 0.0, np.zeros(v.shape[1])
        blocks = range(nblk) if order == 0 else range(nblk - 1, -1, -1)
        for t in blocks:
            js = np.arange(t * bc, min((t + 1) * bc, N))
            js = js[np.isfinite(s[r, js])]
            if js.size == 0:
                continue                        # a block the row cannot see is a no-op
            mp = max(m, float(np.max(s[r, js])))
            a = 0.0 if m == -np.inf else math.exp(m - mp)
            p = np.exp(s[r, js] - mp)
            l = a * l + float(np.sum(p))
            c = _cast(S * p, mode)
            A = a * A + c @ vh[js]
            m = mp
            ns = nonsink[js]
            total[r] += int(np.sum(ns))
            zero[r] += int(np.sum(ns & (c == 0)))
        out[r] = A / (S * l)
    return out, total, zero


def emulate_vectorized(s: np.ndarray, v: np.ndarray, S: float, order: int, mode: str,
                       bc: int = 64, nonsink=None):
    """O2 in closed form: the rescale factors telescope.

    With M(j) the running max just after visiting the block holding key j and
    m the final maximum:  l = sum_j exp(s_j - m),
    A = sum_j cast(S exp(s_j - M(j))) exp(M(j) - m) vhat_j,  O2 = A / (S l).
    """
    S = _scale(S, mode)
    vh = _vhat(v, mode)
    R, N = s.shape
    nonsink = np.ones(N, dtype=bool) if nonsink is None else np.asarray(nonsink, dtype=bool)
    nblk = (N + bc - 1) // bc
    pad = nblk * bc - N
    sp = np.pad(s, ((0, 0), (0, pad)), constant_values=-np.inf)
    bmax = sp.reshape(R, nblk, bc).max(axis=2)              # per-block maxima (-inf if hidden)
    if order == 0:
        run = np.maximum.accumulate(bmax, axis=1)
    else:
        run = np.maximum.accumulate(bmax[:, ::-1], axis=1)[:, ::-1]
    Mj = np.repeat(run, bc, axis=1)[:, :N]                  # running max seen by each key
    m = np.max(s, axis=1, keepdims=True)
    vis = np.isfinite(s)
    with np.errstate(invalid="ignore"):
        p = np.where(vis, np.exp(s - np.where(vis, Mj, 0.0)), 0.0)
        w = np.where(vis, np.exp(np.where(vis, Mj, 0.0) - m), 0.0)
    c = _cast(S * p, mode)
    l = np.sum(np.where(vis, np.exp(s - m), 0.0), axis=1)
    A = (c * w) @ vh
    out = A / (S * l)[:, None]
    ns = vis & nonsink[None, :]
    return out, ns.sum(axis=1).astype(np.int64), (ns & (c == 0)).sum(axis=1).astype(np.int64)


def head_inputs(q_bits, k_bits, v_bits, bias, b: int, h: int, Hq: int, Hkv: int):
    """fp64 q [N,d], k [N,d], v [N,d] of one (batch, q-head); kv head = h // (Hq/Hkv)."""
    g = h // (Hq // Hkv)
    return bf16_to_f64(q_bits[b, h]), bf16_to_f64(k_bits[b, g]), bf16_to_f64(v_bits[b, g])


def attention_oracle(q_bits, k_bits, v_bits, bias, causal: bool, S: float, order: int,
                     mode: str = "kernel", bc: int = 64, sequential: bool = False):
    """O1 and O2 for every row of small bf16 inputs shaped [B,H,N,d].

    Returns (O1 [B,Hq,N,d], O2 [B,Hq,N,d], total [B,Hq,N], zero [B,Hq,N]).
    """
    B, Hq, N, d = q_bits.shape
    Hkv = k_bits.shape[1]
    nonsink = None if bias is None else (np.asarray(bias) == 0)
    o1 = np.zeros((B, Hq, N, d))
    o2 = np.zeros((B, Hq, N, d))
    tot = np.zeros((B, Hq, N), dtype=np.int64)
    zer = np.zeros((B, Hq, N), dtype=np.int64)
    emu = emulate_sequential if sequential else emulate_vectorized
    for b in range(B):
        for h in range(Hq):
            q, k, v = head_inputs(q_bits, k_bits, v_bits, bias, b, h, Hq, Hkv)
            s = logits(q, k, bias, causal)
            o1[b, h] = exact_attention(s, v)
            o2[b, h], tot[b, h], zer[b, h] = emu(s, v, S, order, mode, bc, nonsink)
    return o1, o2, tot, zer

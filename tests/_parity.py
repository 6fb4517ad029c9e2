"""GPU-vs-oracle comparison used by the GPU tests, the smoke check and the bench.

Acceptance (per compared row, 64-row block or case):
* max_c |O_gpu - O2| <= atol + slack_row, where O2 is the oracle's block
  pipeline in kernel mode and slack_row bounds the change of O2 if every E4M3
  (or bf16) rounding decided within a relative 2^-14 of S*p went the other way
  (the GPU's logits and exp2 differ from fp64 by about 1e-6 relative);
  atol = 1e-3 is ten times tighter than the 1e-2 acceptance bound;
* relative MSE against exact attention within 5 % of the oracle's;
* per 64-row block: pair counts equal, underflow counts within the number of
  near-threshold pairs, pooled underflow fraction within 0.5 percentage points;
* bf16 path: max |O_gpu - O1| <= 5e-3.
"""
from __future__ import annotations

import numpy as np

from oracle import core

ATOL = 1e-3
EPS = 2.0 ** -14


def to_gpu_bf16(bits: np.ndarray, device="cuda:0"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def block_rows(B: int, Hq: int, N: int, blocks):
    """Flat row ids of the listed (b, h, r64) blocks, 64 rows each."""
    ids = []
    for b, h, r in blocks:
        base = (b * Hq + h) * N + r * 64
        ids.append(np.arange(base, base + 64, dtype=np.int64))
    return np.concatenate(ids) if ids else np.zeros(0, dtype=np.int64)


def sample_blocks(B: int, Hq: int, N: int, n: int, seed: int):
    """n (b, h, r64) blocks: the first and last block of some heads plus random ones."""
    rng = np.random.default_rng(seed)
    nb = N // 64
    out = {(0, 0, 0), (B - 1, Hq - 1, nb - 1)}
    while len(out) < min(n, B * Hq * nb):
        out.add((int(rng.integers(B)), int(rng.integers(Hq)), int(rng.integers(nb))))
    return sorted(out)


def compare(out_gpu: np.ndarray, stats_gpu, qb, kb, vb, bias, causal, S, order, blocks=None,
            atol: float = ATOL, eps: float = EPS, nthreads: int = 0):
    """Compare GPU results with the oracle on the given blocks (all rows if None).

    out_gpu: [B,Hq,N,d] float array; stats_gpu: [B,Hq,N/64,2] ints or None.
    Returns a report dict; raises AssertionError on a parity failure.
    """
    B, Hq, N, d = qb.shape
    if blocks is None:
        blocks = [(b, h, r) for b in range(B) for h in range(Hq) for r in range(N // 64)]
    ids = block_rows(B, Hq, N, blocks)
    mode = "bf16" if S == 0 else "kernel"
    ref = core.rows(qb, kb, vb, bias, causal, S if S != 0 else 1.0, order, mode, row_ids=ids,
                    eps=eps, want_exact=True, nthreads=nthreads)
    got = out_gpu.reshape(-1, d)[ids].astype(np.float64)
    dev = np.max(np.abs(got - ref["o2"]), axis=1)
    widened = int(np.sum(dev > atol))
    bad = dev > atol + ref["slack"]
    rep = {"rows": int(ids.size), "max_dev": float(dev.max()), "rows_widened": widened,
           "max_dev_exact": float(np.max(np.abs(got - ref["o1"]))),
           "max_o2_exact": float(np.max(np.abs(ref["o2"] - ref["o1"])))}
    assert not np.any(bad), (f"{int(bad.sum())} rows beyond atol+slack; worst dev "
                             f"{dev[bad].max():.3g} slack {ref['slack'][bad][np.argmax(dev[bad])]:.3g}")
    e1 = np.sum(ref["o1"] ** 2)
    rel_gpu = np.sum((got - ref["o1"]) ** 2) / e1
    rel_o2 = np.sum((ref["o2"] - ref["o1"]) ** 2) / e1
    rep["relmse_gpu"], rep["relmse_oracle"] = float(rel_gpu), float(rel_o2)
    assert abs(rel_gpu - rel_o2) <= 0.05 * rel_o2 + 1e-15, f"relMSE {rel_gpu:.4g} vs oracle {rel_o2:.4g}"
    if S == 0:
        assert rep["max_dev_exact"] <= 5e-3, f"bf16 path vs fp64: {rep['max_dev_exact']:.3g}"
    if stats_gpu is not None:
        nblk = len(blocks)
        o_tot = ref["total"].reshape(nblk, 64).sum(axis=1)
        o_zero = ref["zero"].reshape(nblk, 64).sum(axis=1)
        o_amb = ref["zero_amb"].reshape(nblk, 64).sum(axis=1)
        g = np.array([stats_gpu[b, h, r] for (b, h, r) in blocks], dtype=np.int64).reshape(nblk, 2)
        assert np.array_equal(g[:, 0], o_tot), "pair counts differ"
        assert np.all(np.abs(g[:, 1] - o_zero) <= o_amb), "underflow counts differ beyond near ties"
        fg = g[:, 1].sum() / max(g[:, 0].sum(), 1)
        fo = o_zero.sum() / max(o_tot.sum(), 1)
        rep["underflow_gpu"], rep["underflow_oracle"] = float(fg), float(fo)
        assert abs(fg - fo) <= 0.005
    return rep

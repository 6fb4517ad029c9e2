"""GPU-vs-oracle comparison used by the GPU tests, the smoke check and the bench.

Acceptance (per compared row, 64-row block or case):
* max_c |O_gpu - O2| <= atol + slack_row, where O2 is the oracle's block
  pipeline in kernel mode and slack_row bounds the change of O2 if every E4M3
  (or bf16) rounding decided within a relative 2^-14 of S*p went the other way
  (the GPU's logits and exp2 differ from fp64 by about 1e-6 relative);
  atol = 1e-3 is ten times tighter than the 1e-2 acceptance bound; at most
  0.1 % of the rows (and at least one) may need the slack to pass;
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


def widened_allowance(rows: int) -> int:
    """Rows that may exceed atol and pass only through the slack: 0.1 % of the rows
    compared, and at least one (a single flipped sink code widens its row)."""
    return max(1, int(1e-3 * rows))


def to_gpu_bf16(bits: np.ndarray, device="cuda:0"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def block_rows(B: int, Hq: int, N: int, blocks):
    """Flat row ids of the listed (b, h, r64) blocks: 64 rows each, fewer in a partial
    last block (N not a multiple of 64)."""
    ids = []
    for b, h, r in blocks:
        base = (b * Hq + h) * N
        ids.append(np.arange(base + r * 64, base + min(r * 64 + 64, N), dtype=np.int64))
    return np.concatenate(ids) if ids else np.zeros(0, dtype=np.int64)


def stride_blocks(B: int, Hq: int, N: int, stride: int):
    """Every `stride`-th 64-row block of every head, at an offset that moves from head to
    head (so that together the heads cover every residue), plus each head's last block."""
    nb = N // 64
    out = set()
    for b in range(B):
        for h in range(Hq):
            off = ((b * Hq + h) * 7) % stride
            out.update((b, h, r) for r in range(off, nb, stride))
            out.add((b, h, nb - 1))
    return sorted(out)


def sample_blocks(B: int, Hq: int, N: int, n: int, seed: int):
    """n (b, h, r64) blocks: the first and last block of some heads plus random ones."""
    rng = np.random.default_rng(seed)
    nb = N // 64
    out = {(0, 0, 0), (B - 1, Hq - 1, nb - 1)}
    while len(out) < min(n, B * Hq * nb):
        out.add((int(rng.integers(B)), int(rng.integers(Hq)), int(rng.integers(nb))))
    return sorted(out)


# FP8 logits.  Bound on the error of one FP8 dot product on the matrix cores
# relative to the sum of the magnitudes of its products.  Measured on gfx950 for
# 32x32x64 E4M3 products: at most 2^-14.9 (the products are aligned to the
# largest of a group and the bits below about 2^-14 of it are dropped); the bound
# keeps a factor of about 3.7 over that.  Two or more k-steps add in fp32, whose
# rounding is far below this.
ACC_REL = 2.0 ** -13
LOG2E = 1.4426950408889634


def qk8_logit_err(qd_bits, kd_bits, ids):
    """Per row: bound Delta on |logit error| in log2 units, ACC_REL * log2(e)/sqrt(d) *
    max over keys of sum_d |q_d k_d|, on the dequantised Q and K (bf16 bits)."""
    q = _bf16_f64(qd_bits)
    k = _bf16_f64(kd_bits)
    B, Hq, N, d = q.shape
    grp = Hq // k.shape[1]
    out = np.empty(ids.size)
    bh = ids // N
    for key in np.unique(bh):
        sel = np.nonzero(bh == key)[0]
        b, h = divmod(int(key), Hq)
        rows = np.abs(q[b, h][ids[sel] % N])
        out[sel] = np.max(rows @ np.abs(k[b, h // grp]).T, axis=1)
    return ACC_REL * LOG2E / np.sqrt(d) * out


def _bf16_f64(bits):
    return ((np.asarray(bits).astype(np.uint32) & 0xFFFF) << 16).view(np.float32).astype(np.float64)


def compare_qk8(out_gpu, stats_gpu, qd_bits, kd_bits, vb, bias, causal, S, order, blocks=None,
                nthreads: int = 0):
    """compare() for the FP8-logit path, against the oracle on the dequantised Q and K.

    With |logit error| <= Delta (log2 units) in each row, every p and the running
    max move by at most Delta, so p, the running-max weights and l change by a
    relative delta = 2 ln2 Delta at most (the weights telescope to exp2(m_t - m_T)).
    Codes then agree except within a relative delta of a rounding point: slack
    with eps = max delta + 2^-14.  The rest moves O by at most
    2 delta A + delta |O| <= 3 delta A (+ second order), A = sum_j w_j |code_j| |V8_j| / (S l),
    the oracle's output with |V|.  Tolerance per row: atol + slack + 3.5 delta A.
    """
    B, Hq, N, d = qd_bits.shape
    if blocks is None:
        blocks = [(b, h, r) for b in range(B) for h in range(Hq) for r in range((N + 63) // 64)]
    ids = block_rows(B, Hq, N, blocks)
    delta = 2.0 * np.log(2.0) * qk8_logit_err(qd_bits, kd_bits, ids)
    abs_v = np.asarray(vb, dtype=np.uint16) & np.uint16(0x7FFF)
    a = core.rows(qd_bits, kd_bits, abs_v, bias, causal, S, order, "kernel", row_ids=ids,
                  want_exact=False, nthreads=nthreads)["o2"]
    a_row = np.max(np.abs(a), axis=1)
    by_id = dict(zip(ids.tolist(), range(ids.size)))

    def extra(rows):
        sel = np.array([by_id[int(r)] for r in rows])
        return 3.5 * delta[sel] * a_row[sel]

    rep = compare(out_gpu, stats_gpu, qd_bits, kd_bits, vb, bias, causal, S, order, blocks,
                  eps=float(delta.max()) + EPS, nthreads=nthreads, extra=extra)
    rep["logit_err_bound_max"] = float(delta.max() / (2.0 * np.log(2.0)))
    return rep


def compare(out_gpu: np.ndarray, stats_gpu, qb, kb, vb, bias, causal, S, order, blocks=None,
            atol: float = ATOL, eps: float = EPS, nthreads: int = 0, extra=None):
    """Compare GPU results with the oracle on the given blocks (all rows if None).

    out_gpu: [B,Hq,N,d] float array; stats_gpu: [B,Hq,ceil(N/64),2] ints or None.
    extra: optional callable(ids) -> per-row tolerance added to atol + slack.
    Returns a report dict; raises AssertionError on a parity failure.
    """
    B, Hq, N, d = qb.shape
    if blocks is None:
        blocks = [(b, h, r) for b in range(B) for h in range(Hq) for r in range((N + 63) // 64)]
    ids = block_rows(B, Hq, N, blocks)
    mode = "bf16" if S == 0 else "kernel"
    ref = core.rows(qb, kb, vb, bias, causal, S if S != 0 else 1.0, order, mode, row_ids=ids,
                    eps=eps, want_exact=True, nthreads=nthreads)
    got = out_gpu.reshape(-1, d)[ids].astype(np.float64)
    dev = np.max(np.abs(got - ref["o2"]), axis=1)
    widened = int(np.sum(dev > atol))
    tol_extra = np.zeros(ids.size) if extra is None else extra(ids)
    bad = dev > atol + ref["slack"] + tol_extra
    rep = {"rows": int(ids.size), "max_dev": float(dev.max()), "rows_widened": widened,
           "max_dev_exact": float(np.max(np.abs(got - ref["o1"]))),
           "max_o2_exact": float(np.max(np.abs(ref["o2"] - ref["o1"]))),
           "max_dev_over_tol": float(np.max(dev / (atol + ref["slack"] + tol_extra)))}
    assert not np.any(bad), (f"{int(bad.sum())} rows beyond atol+slack; worst dev "
                             f"{dev[bad].max():.3g} slack {ref['slack'][bad][np.argmax(dev[bad])]:.3g} "
                             f"extra {tol_extra[bad][np.argmax(dev[bad])]:.3g}")
    if extra is None:
        assert widened <= widened_allowance(ids.size), f"{widened} of {ids.size} rows needed the slack"
    e1 = np.sum(ref["o1"] ** 2)
    rel_gpu = np.sum((got - ref["o1"]) ** 2) / e1
    rel_o2 = np.sum((ref["o2"] - ref["o1"]) ** 2) / e1
    rep["relmse_gpu"], rep["relmse_oracle"] = float(rel_gpu), float(rel_o2)
    assert abs(rel_gpu - rel_o2) <= 0.05 * rel_o2 + 1e-15, f"relMSE {rel_gpu:.4g} vs oracle {rel_o2:.4g}"
    if S == 0:
        assert rep["max_dev_exact"] <= 5e-3, f"bf16 path vs fp64: {rep['max_dev_exact']:.3g}"
    if stats_gpu is not None:
        nblk = len(blocks)
        # rows per block: 64, or fewer in a partial last block
        starts = np.cumsum([0] + [min(64, N - r * 64) for (_, _, r) in blocks[:-1]])
        o_tot = np.add.reduceat(ref["total"], starts)
        o_zero = np.add.reduceat(ref["zero"], starts)
        o_amb = np.add.reduceat(ref["zero_amb"], starts)
        g = np.array([stats_gpu[b, h, r] for (b, h, r) in blocks], dtype=np.int64).reshape(nblk, 2)
        assert np.array_equal(g[:, 0], o_tot), "pair counts differ"
        assert np.all(np.abs(g[:, 1] - o_zero) <= o_amb), "underflow counts differ beyond near ties"
        fg = g[:, 1].sum() / max(g[:, 0].sum(), 1)
        fo = o_zero.sum() / max(o_tot.sum(), 1)
        rep["underflow_gpu"], rep["underflow_oracle"] = float(fg), float(fo)
        assert abs(fg - fo) <= 0.005
    return rep

"""Pins from above for the oracle's tolerance outputs.

The GPU parity tests accept a row when its deviation from the oracle is within
atol plus the oracle's own allowance for E4M3 rounding decisions that sit near a
rounding point (the P-cast summary, "Ottimizzazione 2": the cast rounds S*p to a
3-bit-mantissa grid whose values at or below 2^-10 become zero).  These tests pin
that allowance to closed forms on hand-built rows, so that an allowance that is too
large (which would make every GPU check vacuous) fails here:

* `slack`: the sum over pairs whose rounding is decided within a relative eps of
  S*p of (grid step there) * exp(M_j - m) * max_c |vhat_jc| / (S l), M_j the
  running max applied to key j and m the final one -- zero when no pair is near a
  rounding point, one grid step times the weights when one pair is;
* `zero_amb`: the number of non-sink pairs whose zero / non-zero decision lies
  within eps of the threshold 2^-10 -- zero or one on these rows;
* the same for the decode oracle (ranges merged by the online-softmax rescale,
  FlashAttention blog "La ricorrenza softmax online") and for the row
  diagnostics' `lost_amb` (the share of non-sink mass whose decision is near the
  threshold).

Rows are built so that every logit is exact in fp64: Q = e_0 (one-hot, bf16 1.0),
K_j = 8 x_j e_0 with d = 64, so q.k_j / sqrt(d) = x_j exactly, and the bias adds
an fp32 value.  A logit that must put S*p on a rounding point is ln(point) rounded
to fp32, which lands within about 1e-7 relative of the point -- far inside eps.
"""
import math

import numpy as np
import pytest

from oracle import core, decode, e4m3, rowdiag

D = 64
EPS = 2.0 ** -14  # the near-tie width the GPU parity tests use


def _bits(x):
    """bf16 bits of values that bf16 holds exactly."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exact in bf16"
    return (u >> 16).astype(np.uint16)


def _row_inputs(x, vrows, Hq=1):
    """Q = e_0 for Hq heads of one row block, K_j = 8 x_j e_0, V rows as given."""
    N = len(x)
    q = np.zeros((1, Hq, N, D), dtype=np.float32)
    q[..., 0] = 1.0
    k = np.zeros((1, 1, N, D), dtype=np.float32)
    k[0, 0, :, 0] = 8.0 * np.asarray(x, dtype=np.float32)
    v = np.asarray(vrows, dtype=np.float32).reshape(1, 1, N, D)
    return _bits(q), _bits(k), _bits(v)


def _v_rows(N, special=None):
    """V = 1.0 everywhere, except rows given as {j: (value at column 0, value at column 1)}."""
    v = np.ones((N, D), dtype=np.float32)
    for j, (a, b) in (special or {}).items():
        v[j, 0], v[j, 1] = a, b
    return v


def _last_row(r):
    """Oracle outputs of the last row of a core.rows result."""
    return {k: np.asarray(val)[-1] for k, val in r.items()}


def _f32(x):
    return float(np.float32(x))


# ---------------------------------------------------------------------------
# C core (O2 of the P-cast path)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("S", [1.0, 256.0, 448.0])
@pytest.mark.parametrize("order", [0, 1])
def test_core_no_pair_near_a_rounding_point(S, order):
    """Every S*p on the grid or far from its midpoints: slack and zero_amb are 0."""
    N = 128
    x = np.zeros(N)
    x[70] = 2.0                      # block 1 raises the max to 2: S*e^-2 is no grid midpoint
    bias = np.zeros(N, dtype=np.float32)
    q, k, v = _row_inputs(x, _v_rows(N, {5: (3.0, -2.75)}))
    r = core.rows(q, k, v, bias, False, S, order, "kernel", eps=EPS)
    for t in (S * math.exp(-2.0),):  # the one off-grid value: check it is not near a midpoint
        lo, hi = e4m3.e4m3_rne(t * (1 - EPS)), e4m3.e4m3_rne(t * (1 + EPS))
        assert lo == hi
    assert np.all(r["slack"] == 0.0)
    assert np.all(r["zero_amb"] == 0)


@pytest.mark.parametrize("S", [1.0, 256.0])
def test_core_one_midpoint_pair_single_block(S):
    """One key with S*p on the midpoint between two E4M3 values: slack = step * max|vhat| / (S l)."""
    N = 64
    point = 0.53125                  # midpoint of 0.5 and 0.5625 (step 2^-4 in [0.5, 1))
    b = _f32(math.log(point / S))
    x = np.zeros(N)
    bias = np.zeros(N, dtype=np.float32)
    bias[10] = b
    q, k, v = _row_inputs(x, _v_rows(N, {10: (3.0, -2.75)}))
    r = _last_row(core.rows(q, k, v, bias, False, S, 0, "kernel", eps=EPS))
    p = math.exp(b)
    assert abs(S * p - point) < 1e-6 * point
    l = 63.0 + p
    expect = 0.0625 * 3.0 / (S * l)
    assert r["slack"] == pytest.approx(expect, rel=1e-14)
    assert r["zero_amb"] == 0        # a midpoint far from 2^-10 decides no zero


def test_core_one_midpoint_pair_under_a_later_max():
    """Forward order, the midpoint key in block 0 and the row max (2) in block 1:
    the pair's step is weighted by exp(M_j - m) = e^-2 and l carries the rescale."""
    N = 128
    point = 0.53125
    b = _f32(math.log(point))
    x = np.zeros(N)
    x[100] = 2.0
    bias = np.zeros(N, dtype=np.float32)
    bias[10] = b
    q, k, v = _row_inputs(x, _v_rows(N, {10: (3.0, -2.75)}))
    r = _last_row(core.rows(q, k, v, bias, False, 1.0, 0, "kernel", eps=EPS))
    p = math.exp(b)
    e2 = math.exp(-2.0)
    l = (63.0 + p) * e2 + (63.0 * e2 + 1.0)
    expect = 0.0625 * e2 * 3.0 / l
    assert r["slack"] == pytest.approx(expect, rel=1e-14)
    # reverse order sees the max first: the key's S*p = p e^-2 is no longer on a midpoint
    rr = _last_row(core.rows(q, k, v, bias, False, 1.0, 1, "kernel", eps=EPS))
    assert rr["slack"] == 0.0


def test_core_one_pair_at_the_zero_threshold():
    """The only non-sink key has S*p = 2^-10 (to fp32): zero_amb = 1, and its slack is one
    step 2^-9 times max|vhat| / (S l); the sinks (bias != 0) sit at p = 1, on the grid."""
    N = 64
    b0 = _f32(10.0 * math.log(2.0))
    bias = np.full(N, b0, dtype=np.float32)
    bias[7] = 0.0                    # key 7: logit 0, p = e^-b0 ~ 2^-10
    x = np.zeros(N)
    q, k, v = _row_inputs(x, _v_rows(N, {7: (-1.5, 0.5)}))
    r = _last_row(core.rows(q, k, v, bias, False, 1.0, 0, "kernel", eps=EPS))
    p = math.exp(-b0)
    assert abs(p - 2.0 ** -10) < 1e-6 * 2.0 ** -10
    assert r["total"] == 1 and r["zero_amb"] == 1
    assert r["zero"] == int(e4m3.e4m3_rne(p) == 0.0)
    l = 63.0 + p
    assert r["slack"] == pytest.approx(2.0 ** -9 * 1.5 / l, rel=1e-14)


def test_core_eps_sets_the_width():
    """A pair 2^-13 (relative) above a midpoint is near for eps = 2^-12, not for 2^-14."""
    N = 64
    point = 0.53125 * (1 + 2.0 ** -13)
    b = _f32(math.log(point))
    bias = np.zeros(N, dtype=np.float32)
    bias[3] = b
    q, k, v = _row_inputs(np.zeros(N), _v_rows(N))
    wide = _last_row(core.rows(q, k, v, bias, False, 1.0, 0, "kernel", eps=2.0 ** -12))
    narrow = _last_row(core.rows(q, k, v, bias, False, 1.0, 0, "kernel", eps=2.0 ** -14))
    assert wide["slack"] == pytest.approx(0.0625 / (63.0 + math.exp(b)), rel=1e-14)
    assert narrow["slack"] == 0.0


# ---------------------------------------------------------------------------
# Decode oracle (split KV, ranges merged)
# ---------------------------------------------------------------------------

def _decode_inputs(x, bias, special):
    q, k, v = _row_inputs(x, _v_rows(len(x), special))
    return q[:, :, -1:, :], k, v     # one decode row at the last position: it sees every key


def test_decode_no_pair_near_a_rounding_point():
    N = 128
    x = np.zeros(N)
    x[70] = 2.0
    bias = np.zeros(N, dtype=np.float32)
    q, k, v = _decode_inputs(x, bias, {5: (3.0, -2.75)})
    for split in (64, 128):
        for order in (0, 1):
            r = decode.rows(q, k, v, bias, 256.0, order, split, eps=EPS)
            assert r["slack"].item() == 0.0 and r["zero_amb"].item() == 0


@pytest.mark.parametrize("split", [64, 128])
def test_decode_one_midpoint_pair(split):
    """The midpoint key in keys 0..63, the max (2) in keys 64..127.  One range: forward
    order as in the core.  Two ranges of 64: range 0 keeps its own max 0 and the merge
    weights it by e^-2 -- the same closed form."""
    N = 128
    point = 0.53125
    b = _f32(math.log(point))
    x = np.zeros(N)
    x[100] = 2.0
    bias = np.zeros(N, dtype=np.float32)
    bias[10] = b
    q, k, v = _decode_inputs(x, bias, {10: (3.0, -2.75)})
    r = decode.rows(q, k, v, bias, 1.0, 0, split, eps=EPS)
    p, e2 = math.exp(b), math.exp(-2.0)
    l = (63.0 + p) * e2 + (63.0 * e2 + 1.0)
    assert r["slack"].item() == pytest.approx(0.0625 * e2 * 3.0 / l, rel=1e-14)
    assert r["zero_amb"].item() == 0


def test_decode_one_pair_at_the_zero_threshold():
    N = 64
    b0 = _f32(10.0 * math.log(2.0))
    bias = np.full(N, b0, dtype=np.float32)
    bias[7] = 0.0
    q, k, v = _decode_inputs(np.zeros(N), bias, {7: (-1.5, 0.5)})
    r = decode.rows(q, k, v, bias, 1.0, 0, 64, eps=EPS)
    p = math.exp(-b0)
    assert r["total"].item() == 1 and r["zero_amb"].item() == 1
    assert r["slack"].item() == pytest.approx(2.0 ** -9 * 1.5 / (63.0 + p), rel=1e-14)


# ---------------------------------------------------------------------------
# Row diagnostics: lost_amb
# ---------------------------------------------------------------------------

def test_rowdiag_lost_amb_closed_form():
    """Two non-sink keys: key 7 at p = 2^-10 (on the threshold), key 9 at p = e^-1 2^-10
    (far below it); the rest are sinks at p = 1.  lost_amb = w_7 / (w_7 + w_9) =
    1 / (1 + e^-1); with key 7 moved off the threshold it is 0."""
    N = 64
    b0 = _f32(10.0 * math.log(2.0))
    bias = np.full(N, b0, dtype=np.float32)
    bias[7] = bias[9] = 0.0
    x = np.zeros(N)
    x[9] = -1.0
    q, k, _ = _row_inputs(x, _v_rows(N))
    r = rowdiag.rows(q, k, bias, False, 1.0, 0, row_ids=[N - 1], eps=EPS)
    assert r["lost_amb"][0] == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-14)
    w7, w9 = math.exp(-b0), math.exp(-1.0 - b0)
    lost = (w9 + (w7 if e4m3.e4m3_rne(w7) == 0.0 else 0.0)) / (w7 + w9)
    assert r["lost"][0] == pytest.approx(lost, rel=1e-14)
    x[7] = 0.5                       # key 7 at 2^-10 e^0.5: a non-zero code, nothing near
    q, k, _ = _row_inputs(x, _v_rows(N))
    r = rowdiag.rows(q, k, bias, False, 1.0, 0, row_ids=[N - 1], eps=EPS)
    assert r["lost_amb"][0] == 0.0

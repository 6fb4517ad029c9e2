"""Pins for the FP8-logits extension of the oracle (Q and K in E4M3 with
power-of-two block scales: one per query row, one per 64-key block).

What pins it:
* the scale rule against its definition by brute force (smallest e with
  max|x| <= 448 * 2^e), at the boundaries 448 * 2^k and between them, and the
  array form against the scalar one;
* quantised values lie on the scaled E4M3 grid, never saturate, are exactly
  bf16-representable, are the RNE points, and quantising twice changes nothing;
* blocks are independent: scaling one block by 2^k moves its exponent by k and
  leaves every other block as it was;
* Q and K already on the E4M3 grid with max|x| = 448 in every block quantise to
  themselves, so the oracle's output is unchanged bit for bit;
* the logits computed from the quantised tensors equal the sum of E4M3 code
  products times 2^(e_i + e_block(j)) / sqrt(d), written out by hand;
* planted mistakes (no scale; one scale per head) fail the pins.
"""
import math

import numpy as np
import pytest

import synthetic
from oracle import core, e4m3, qk8, reference


@pytest.mark.parametrize("k", range(-30, 12))
def test_scale_exp_boundaries(k):
    edge = 448.0 * 2.0 ** k
    assert qk8.head_scale_exp(edge) == k
    assert qk8.head_scale_exp(np.nextafter(edge, np.inf)) == k + 1
    assert qk8.head_scale_exp(np.nextafter(edge, 0.0)) == k
    assert qk8.head_scale_exp(0.75 * edge) == k          # between 2^(k-1)*448 and 2^k*448


def test_scale_exp_definition_random():
    rng = np.random.default_rng(0)
    for a in np.exp(rng.uniform(-40, 20, 5000)):
        e = qk8.head_scale_exp(a)
        assert a <= 448.0 * 2.0 ** e and a > 448.0 * 2.0 ** (e - 1)
    assert qk8.head_scale_exp(0.0) == 0


def test_scale_exps_matches_scalar_rule():
    rng = np.random.default_rng(5)
    a = np.concatenate([np.exp(rng.uniform(-40, 20, 3000)), [0.0],
                        448.0 * 2.0 ** np.arange(-20, 10.0), np.nextafter(448.0 * 2.0 ** np.arange(-20, 10.0), 1e9)])
    assert np.array_equal(qk8.scale_exps(a), [qk8.head_scale_exp(x) for x in a])


@pytest.mark.parametrize("rows", [1, 64, 256])
def test_quantised_values_on_scaled_grid(rows):
    q, _, _ = synthetic.qkv_bf16(2, 3, 3, 256, 64, 41)
    qq, exps = qk8.quantize_blocks(q, rows)
    assert exps.shape == (2, 3, 256 // rows)
    x = reference.bf16_to_f64(q)
    y = reference.bf16_to_f64(qq)
    grid = e4m3.grid()
    for b in range(2):
        for h in range(3):
            for r in range(256 // rows):
                sl = slice(r * rows, (r + 1) * rows)
                e = int(exps[b, h, r])
                amax = np.max(np.abs(x[b, h, sl]))
                assert amax <= 448.0 * 2.0 ** e and amax > 448.0 * 2.0 ** (e - 1)
                z = np.abs(np.ldexp(y[b, h, sl], -e))
                assert z.max() <= 448.0
                assert np.all(np.isin(z, grid))
                # the nearest grid point: |x/2^e - z| is at most half a grid step
                assert np.array_equal(np.ldexp(y[b, h, sl], -e), e4m3.e4m3_rne(np.ldexp(x[b, h, sl], -e)))
    # quantising again changes no value; a block's exponent drops by one exactly
    # when its max rounded down onto 448 * 2^(e-1)
    q2, e2 = qk8.quantize_blocks(qq, rows)
    assert np.array_equal(q2, qq)
    ymax = np.max(np.abs(y.reshape(2, 3, 256 // rows, -1)), axis=3)
    drop = e2 != exps
    assert np.all(e2[drop] == exps[drop] - 1)
    assert np.all(ymax[drop] == 448.0 * 2.0 ** (exps[drop] - 1.0))


def test_named_granularities():
    q, k, _ = synthetic.qkv_bf16(1, 2, 2, 128, 64, 45)
    assert qk8.Q_BLOCK_ROWS == 1 and qk8.K_BLOCK_ROWS == 64
    for f, rows in ((qk8.quantize_q, 1), (qk8.quantize_k, 64)):
        a, ea = f(q)
        b, eb = qk8.quantize_blocks(q, rows)
        assert np.array_equal(a, b) and np.array_equal(ea, eb)


@pytest.mark.parametrize("rows", [1, 64])
def test_blocks_are_independent(rows):
    q, _, _ = synthetic.qkv_bf16(1, 2, 2, 256, 64, 46)
    base, e0 = qk8.quantize_blocks(q, rows)
    x = reference.bf16_to_f64(q).copy()
    blk = 1 if rows == 64 else 77                  # one block of head 1
    sl = slice(blk * rows, (blk + 1) * rows)
    x[0, 1, sl] *= 2.0 ** 9
    bits = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    moved, e1 = qk8.quantize_blocks(bits, rows)
    diff = e1 - e0
    assert diff[0, 1, blk] == 9 and np.count_nonzero(diff) == 1
    y0, y1 = reference.bf16_to_f64(base), reference.bf16_to_f64(moved)
    assert np.array_equal(y1[0, 1, sl], y0[0, 1, sl] * 2.0 ** 9)
    y1[0, 1, sl] = y0[0, 1, sl]
    assert np.array_equal(y1, y0)


def test_partial_last_block_is_its_existing_rows():
    """N = 100: the last 64-key block holds keys 64..99; its scale and values equal those of
    that block quantised on its own (a plain 36-row block of the same rows), and the full
    block before it is unchanged by the cut."""
    k, _, _ = synthetic.qkv_bf16(1, 2, 2, 100, 64, 47)
    got, e = qk8.quantize_blocks(k, 64)
    assert e.shape == (1, 2, 2)
    tail, et = qk8.quantize_blocks(np.ascontiguousarray(k[:, :, 64:]), 36)
    assert np.array_equal(got[:, :, 64:], tail) and np.array_equal(e[..., 1], et[..., 0])
    head, eh = qk8.quantize_blocks(np.ascontiguousarray(k[:, :, :64]), 64)
    assert np.array_equal(got[:, :, :64], head) and np.array_equal(e[..., 0], eh[..., 0])


def test_rotated_values_partial_last_block():
    """quantize_values (the rotated path's quantiser) on N = 100 rows: the partial block equals
    its 36 rows quantised on their own, the full block is unchanged by the cut."""
    q, _, _ = synthetic.qkv_bf16(1, 2, 2, 100, 64, 48)
    x = qk8.rotate(q, np.where(np.arange(64) % 3 == 0, -1.0, 1.0))
    got, e = qk8.quantize_values(x, 64)
    tail, et = qk8.quantize_values(np.ascontiguousarray(x[:, :, 64:]), 36)
    head, eh = qk8.quantize_values(np.ascontiguousarray(x[:, :, :64]), 64)
    assert np.array_equal(got[:, :, 64:], tail) and np.array_equal(e[..., 1], et[..., 0])
    assert np.array_equal(got[:, :, :64], head) and np.array_equal(e[..., 0], eh[..., 0])


def test_grid_inputs_unchanged():
    """Q, K drawn from the E4M3 grid with max |x| = 448 in every row: quantisation
    is the identity at both granularities."""
    rng = np.random.default_rng(1)
    grid = e4m3.grid()
    shape = (1, 2, 128, 64)
    vals = rng.choice(np.concatenate([-grid, grid]), size=shape)
    vals[..., 0] = 448.0
    bits = (vals.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    qq, eq = qk8.quantize_q(bits)
    kq, ek = qk8.quantize_k(bits)
    assert np.array_equal(qq, bits) and np.all(eq == 0)
    assert np.array_equal(kq, bits) and np.all(ek == 0)
    _, _, v = synthetic.qkv_bf16(1, 2, 2, 128, 64, 42)
    bias = synthetic.sink_bias(128, 7.0)
    a = core.rows(bits, bits, v, bias, True, 256.0, 1, "kernel")
    b = core.rows(qq, kq, v, bias, True, 256.0, 1, "kernel")
    assert np.array_equal(a["o2"], b["o2"]) and np.array_equal(a["zero"], b["zero"])


def test_logits_are_scaled_code_products():
    q, k, _ = synthetic.qkv_bf16(1, 1, 1, 128, 32, 43)
    xq = reference.bf16_to_f64(q).copy()
    xk = reference.bf16_to_f64(k).copy()
    xq[0, 0, ::3] *= 2.0 ** -5                    # rows at different scales
    xk[0, 0, 64:] *= 2.0 ** 6                     # the second key block larger
    q = (xq.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    k = (xk.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    qq, eq = qk8.quantize_q(q)
    kq, ek = qk8.quantize_k(k)
    assert len(set(eq[0, 0].tolist())) > 1 and ek[0, 0, 1] - ek[0, 0, 0] >= 5
    s = reference.logits(reference.bf16_to_f64(qq[0, 0]), reference.bf16_to_f64(kq[0, 0]), None, False)
    # by hand: decode the E4M3 codes, multiply, sum, then scale
    rows = [0, 1, 5, 63, 64, 127]
    for i in rows:
        cq = e4m3.e4m3_encode(np.ldexp(xq[0, 0, i], -int(eq[0, 0, i])))
        for j in rows:
            ck = e4m3.e4m3_encode(np.ldexp(xk[0, 0, j], -int(ek[0, 0, j // 64])))
            acc = 0.0
            for c in range(32):
                acc += e4m3.DECODE_TABLE[cq[c]] * e4m3.DECODE_TABLE[ck[c]]
            expect = acc * 2.0 ** (int(eq[0, 0, i]) + int(ek[0, 0, j // 64])) / math.sqrt(32)
            assert abs(s[i, j] - expect) <= 1e-12 * max(1.0, abs(expect))


def test_planted_missing_scale_is_caught():
    q, _, _ = synthetic.qkv_bf16(1, 1, 1, 64, 32, 44)
    x = reference.bf16_to_f64(q)
    wrong = e4m3.e4m3_rne(x)                 # no scale: |x| < 448 so nothing saturates,
    qq, _ = qk8.quantize_q(q)                # but the grid is far too coarse near zero
    assert not np.array_equal(wrong, reference.bf16_to_f64(qq))


def test_planted_head_scale_is_caught():
    """One scale for the whole head instead of one per row: rows far below the
    head's max fall into E4M3's subnormal range and lose precision."""
    q, _, _ = synthetic.qkv_bf16(1, 1, 1, 64, 32, 47)
    x = reference.bf16_to_f64(q).copy()
    x[0, 0, 1::2] *= 2.0 ** -16
    bits = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    per_head, _ = qk8.quantize_blocks(bits, 64)
    per_row, _ = qk8.quantize_q(bits)
    err_head = np.abs(reference.bf16_to_f64(per_head) - x)[0, 0, 1::2]
    err_row = np.abs(reference.bf16_to_f64(per_row) - x)[0, 0, 1::2]
    assert not np.array_equal(per_head, per_row)
    # per row: relative error at most 2^-4 (3 mantissa bits, no subnormals at these maxima)
    assert np.all(err_row <= 2.0 ** -4 * np.abs(x[0, 0, 1::2]) + 1e-300)
    assert np.sum(err_head ** 2) > 100 * np.sum(err_row ** 2)


# ---- random rotation (randomised Hadamard transform) ----

@pytest.mark.parametrize("d", [1, 2, 8, 64, 128])
def test_hadamard_is_orthogonal_up_to_d(d):
    h = qk8.hadamard(d)
    assert np.array_equal(h @ h.T, d * np.eye(d))
    assert set(np.unique(h)) <= {-1.0, 1.0}


def test_rotation_keeps_dot_products_exactly():
    q, k, _ = synthetic.qkv_bf16(1, 1, 1, 16, 128, 48)
    signs = np.random.default_rng(3).choice([-1.0, 1.0], size=128)
    rq, rk = qk8.rotate(q, signs)[0, 0], qk8.rotate(k, signs)[0, 0]
    x, y = reference.bf16_to_f64(q)[0, 0], reference.bf16_to_f64(k)[0, 0]
    assert np.array_equal(rq @ rk.T, 128 * (x @ y.T))


def test_rotation_spreads_an_outlier():
    """One large channel becomes +-A on every coordinate (the point of the rotation)."""
    x = np.zeros((1, 1, 1, 64), dtype=np.float32)
    x[..., 5] = 96.0
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    signs = np.ones(64)
    r = qk8.rotate(bits, signs)
    assert np.array_equal(np.abs(r), np.full((1, 1, 1, 64), 96.0))


def test_rotated_quantisation_gives_scaled_logits():
    q, k, _ = synthetic.qkv_bf16(1, 1, 1, 128, 64, 49)
    signs = np.random.default_rng(4).choice([-1.0, 1.0], size=64)
    qb, kb, eq, ek = qk8.quantize_rotated(q, k, signs)
    rq, rk = qk8.rotate(q, signs)[0, 0], qk8.rotate(k, signs)[0, 0]
    dq = reference.bf16_to_f64(qb)[0, 0]
    dk = reference.bf16_to_f64(kb)[0, 0] * 64
    # each value is its rotated input rounded to E4M3 at its block's scale
    for i in (0, 17, 127):
        e = int(eq[0, 0, i])
        assert np.array_equal(dq[i], np.ldexp(e4m3.e4m3_rne(np.ldexp(rq[i], -e)), e))
        e = int(ek[0, 0, i // 64])
        assert np.array_equal(dk[i], np.ldexp(e4m3.e4m3_rne(np.ldexp(rk[i], -e)), e))
    # and the plain dot product of the returned tensors approximates the original one
    x, y = reference.bf16_to_f64(q)[0, 0], reference.bf16_to_f64(k)[0, 0]
    got = reference.bf16_to_f64(qb)[0, 0] @ reference.bf16_to_f64(kb)[0, 0].T
    assert np.max(np.abs(got - x @ y.T)) < 0.2 * np.max(np.abs(x @ y.T))


def test_rotation_lowers_the_error_with_outlier_channels():
    """Gaussian Q, K with four channels 30x larger: without rotation the outliers set
    every row's scale and the small channels lose precision; rotated, the error of
    the logits drops (the FA3 section reports 2.6x on its data)."""
    rng = np.random.default_rng(5)
    q, k, _ = synthetic.qkv_bf16(1, 1, 1, 256, 128, 50)
    x = reference.bf16_to_f64(q).copy()
    y = reference.bf16_to_f64(k).copy()
    for t in (x, y):
        t[..., [3, 40, 77, 100]] *= 30.0
    qbits = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    kbits = (y.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    exact = reference.bf16_to_f64(qbits)[0, 0] @ reference.bf16_to_f64(kbits)[0, 0].T
    qa, _ = qk8.quantize_q(qbits)
    ka, _ = qk8.quantize_k(kbits)
    plain = reference.bf16_to_f64(qa)[0, 0] @ reference.bf16_to_f64(ka)[0, 0].T
    signs = rng.choice([-1.0, 1.0], size=128)
    qr, kr, _, _ = qk8.quantize_rotated(qbits, kbits, signs)
    rot = reference.bf16_to_f64(qr)[0, 0] @ reference.bf16_to_f64(kr)[0, 0].T
    e_plain = np.sqrt(np.mean((plain - exact) ** 2))
    e_rot = np.sqrt(np.mean((rot - exact) ** 2))
    assert e_rot < e_plain

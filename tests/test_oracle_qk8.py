"""Pins for the FP8-logits extension of the oracle (Q and K in E4M3 with a
per-head power-of-two scale).

What pins it:
* the scale rule against its definition by brute force (smallest e with
  max|x| <= 448 * 2^e), at the boundaries 448 * 2^k and between them;
* quantised values lie on the scaled E4M3 grid, never saturate, are exactly
  bf16-representable, and quantising twice changes nothing;
* Q and K already on the E4M3 grid with max|x| = 448 quantise to themselves, so
  the oracle's output is unchanged bit for bit;
* the logits computed from the quantised tensors equal the sum of E4M3 code
  products times 2^(e_q + e_k) / sqrt(d), written out by hand on a small case;
* a planted mistake (dropping the scale) fails the round-trip pin.
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


def test_quantised_values_on_scaled_grid():
    q, _, _ = synthetic.qkv_bf16(2, 3, 3, 256, 64, 41)
    qq, exps = qk8.quantize_heads(q)
    x = reference.bf16_to_f64(q)
    y = reference.bf16_to_f64(qq)
    grid = e4m3.grid()
    for b in range(2):
        for h in range(3):
            e = int(exps[b, h])
            assert np.max(np.abs(x[b, h])) <= 448.0 * 2.0 ** e
            z = np.abs(np.ldexp(y[b, h], -e))
            assert z.max() <= 448.0
            assert np.all(np.isin(z, grid))
            # the nearest grid point: |x/2^e - z| is at most half a grid step
            assert np.array_equal(np.ldexp(y[b, h], -e), e4m3.e4m3_rne(np.ldexp(x[b, h], -e)))
    q2, e2 = qk8.quantize_heads(qq)
    assert np.array_equal(q2, qq) and np.array_equal(e2, exps)


def test_grid_inputs_unchanged():
    """Q, K drawn from the E4M3 grid with max |x| = 448: quantisation is the identity."""
    rng = np.random.default_rng(1)
    grid = e4m3.grid()
    shape = (1, 2, 128, 64)
    vals = rng.choice(np.concatenate([-grid, grid]), size=shape)
    vals[..., 0, 0] = 448.0
    bits = (vals.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    qq, exps = qk8.quantize_heads(bits)
    assert np.array_equal(qq, bits) and np.all(exps == 0)
    _, _, v = synthetic.qkv_bf16(1, 2, 2, 128, 64, 42)
    bias = synthetic.sink_bias(128, 7.0)
    a = core.rows(bits, bits, v, bias, True, 256.0, 1, "kernel")
    b = core.rows(qq, qq, v, bias, True, 256.0, 1, "kernel")
    assert np.array_equal(a["o2"], b["o2"]) and np.array_equal(a["zero"], b["zero"])


def test_logits_are_scaled_code_products():
    q, k, _ = synthetic.qkv_bf16(1, 1, 1, 16, 32, 43)
    qq, eq = qk8.quantize_heads(q)
    kq, ek = qk8.quantize_heads(k)
    s = reference.logits(reference.bf16_to_f64(qq[0, 0]), reference.bf16_to_f64(kq[0, 0]), None, False)
    # by hand: decode the E4M3 codes, multiply, sum, then scale
    cq = e4m3.e4m3_encode(np.ldexp(reference.bf16_to_f64(q[0, 0]), -int(eq[0, 0])))
    ck = e4m3.e4m3_encode(np.ldexp(reference.bf16_to_f64(k[0, 0]), -int(ek[0, 0])))
    dq, dk = e4m3.DECODE_TABLE[cq], e4m3.DECODE_TABLE[ck]
    for i in range(16):
        for j in range(16):
            acc = 0.0
            for c in range(32):
                acc += dq[i, c] * dk[j, c]
            expect = acc * 2.0 ** (int(eq[0, 0]) + int(ek[0, 0])) / math.sqrt(32)
            assert abs(s[i, j] - expect) <= 1e-12 * max(1.0, abs(expect))


def test_planted_missing_scale_is_caught():
    q, _, _ = synthetic.qkv_bf16(1, 1, 1, 64, 32, 44)
    x = reference.bf16_to_f64(q)
    wrong = e4m3.e4m3_rne(x)                 # no per-head scale: |x| < 448 so nothing saturates,
    qq, _ = qk8.quantize_heads(q)            # but the grid is far too coarse near zero
    assert not np.array_equal(wrong, reference.bf16_to_f64(qq))

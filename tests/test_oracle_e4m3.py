"""Pins for the oracle's software E4M3 and bf16 roundings.

What pins them (none of it is the oracle re-deriving itself):
* the format facts the P-cast summary prints (3-bit mantissa, 448 the largest
  value, 2^-10 the round-to-zero threshold) -- tests/golden/pages_facts.json;
* an independent implementation: torch's float8_e4m3fn decode of all 256 codes
  and its cast (which is RNE but not saturating, so only |x| <= 464 is compared);
* brute force: nearest grid point with ties to the even code, by search.
"""
import numpy as np
import pytest
import torch

from oracle import core, e4m3


def test_decode_table_matches_format_facts(golden):
    t = e4m3.DECODE_TABLE
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.sum(np.isfinite(t)) == 254
    assert t[0x7E] == 448.0 == np.nanmax(t)
    assert t[0x01] == 2.0 ** -9 and t[0x08] == 2.0 ** -6
    assert t[0x00] == 0.0 and np.signbit(t[0x80])
    assert len(e4m3.grid()) == 127
    # 3 mantissa bits: 8 grid points in every normal binade
    g = e4m3.grid()
    for E in range(-6, 8):
        assert np.sum((g >= 2.0 ** E) & (g < 2.0 ** (E + 1))) == 2 ** golden["e4m3_mantissa_bits"]["value"]


def test_decode_table_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = e4m3.DECODE_TABLE
    assert np.array_equal(np.isnan(ref), np.isnan(ours))
    fin = np.isfinite(ref)
    assert np.array_equal(ref[fin], ours[fin])
    assert np.array_equal(np.signbit(ref[fin]), np.signbit(ours[fin]))


def test_encode_decode_round_trip():
    fin = [c for c in range(256) if np.isfinite(e4m3.DECODE_TABLE[c])]
    vals = e4m3.DECODE_TABLE[fin]
    assert np.array_equal(e4m3.e4m3_rne(vals), vals)
    assert np.array_equal(e4m3.e4m3_encode(vals)[vals != 0], np.array(fin, dtype=np.uint8)[vals != 0])


def test_zero_threshold(golden):
    thr = golden["e4m3_zero_threshold"]["value"]
    assert thr == 2.0 ** -10
    assert e4m3.e4m3_rne(thr) == 0.0                                  # tie -> even code 0
    assert e4m3.e4m3_rne(np.nextafter(np.float32(thr), np.float32(1))) == 2.0 ** -9
    assert e4m3.e4m3_rne(3 * 2.0 ** -10) == 2.0 ** -8                 # tie between codes 1 and 2 -> 2
    assert e4m3.e4m3_rne(5 * 2.0 ** -10) == 2.0 ** -8                 # tie between codes 2 and 3 -> 2
    # 6.93 is 10 ln 2 to the printed precision
    assert abs(10 * np.log(2) - golden["threshold_log_constant"]["value"]) < 5e-3


def test_saturation(golden):
    assert e4m3.e4m3_rne(448.0) == 448.0
    assert e4m3.e4m3_rne(463.9) == 448.0
    assert e4m3.e4m3_rne(golden["scale_512_overflows"]["value"]) == 448.0
    assert e4m3.e4m3_rne(1e30) == 448.0 and e4m3.e4m3_rne(-1e30) == -448.0
    assert e4m3.e4m3_rne(432.0) == 448.0      # midpoint of 416 (odd code) and 448 (even) -> 448
    assert e4m3.e4m3_rne(400.0) == 384.0      # midpoint of 384 (even code) and 416 (odd) -> 384


def test_rne_brute_force():
    """Nearest grid point by exhaustive search, ties to the even code."""
    g = e4m3.grid()
    codes = np.arange(127)
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.uniform(0, 448, 20000),
        np.exp2(rng.uniform(-14, 8.8, 20000)),
        (g[:-1] + g[1:]) / 2,                   # every midpoint (ties)
        g,
    ])
    x = x[x <= 448]
    d = np.abs(x[:, None] - g[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = np.where(d == best, codes[None, :], 10 ** 6)
    # among equally near codes choose the even one
    even = np.where((cand % 2 == 0) & (cand < 10 ** 6), cand, 10 ** 6).min(axis=1)
    pick = np.where(even < 10 ** 6, even, cand.min(axis=1))
    expect = g[pick]
    assert np.array_equal(e4m3.e4m3_rne(x), expect)
    assert np.array_equal(e4m3.e4m3_rne(-x), -expect)


def test_rne_matches_torch_dense_fp32():
    """Every fp32 with exponent in [-12, -5), and a stride sample of [2^-5, 464]."""
    lo = np.float32(2.0 ** -12).view(np.uint32)
    hi = np.float32(2.0 ** -5).view(np.uint32)
    a = np.arange(lo, hi, dtype=np.uint32).view(np.float32)
    b = np.arange(hi, np.float32(464.0).view(np.uint32), 97, dtype=np.uint32).view(np.float32)
    x = np.concatenate([a, b])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(e4m3.e4m3_rne(x.astype(np.float64)), ref)


def test_c_and_numpy_roundings_agree():
    rng = np.random.default_rng(1)
    x = np.concatenate([np.exp2(rng.uniform(-40, 12, 200000)) * rng.choice([-1, 1], 200000),
                        (e4m3.grid()[:-1] + e4m3.grid()[1:]) / 2, [0.0, 448.0, 500.0]])
    assert np.array_equal(core.e4m3_rne(x), e4m3.e4m3_rne(x))
    assert np.array_equal(core.bf16_rne(x), e4m3.bf16_rne(x))


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(2)
    x = np.exp2(rng.uniform(-30, 10, 200000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(e4m3.bf16_rne(x.astype(np.float64)), ref)


@pytest.mark.parametrize("k", range(10))
def test_pow2_scaling_is_exact_in_fp32(k):
    """x S and / S are exact in fp32 for S = 2^k (P-cast summary, Ottimizzazione 2 point 1)."""
    rng = np.random.default_rng(k)
    p = np.concatenate([rng.uniform(0, 1, 100000), np.exp2(rng.uniform(-126, 0, 100000))]).astype(np.float32)
    S = np.float32(2.0 ** k)
    y = p * S
    assert np.array_equal(y, np.ldexp(p, k).astype(np.float32))
    assert np.array_equal(y / S, p)


def test_scale_448_is_not_exact():
    rng = np.random.default_rng(3)
    p = rng.uniform(0, 1, 100000).astype(np.float32)
    S = np.float32(448.0)
    assert np.sum((p * S) / S != p) > 1000


def test_dp_sawtooth(golden):
    for k in range(9):
        assert e4m3.quant_step_max(2.0 ** k) == golden["dp_pow2"]["value"]
    r = e4m3.quant_step_max(448.0) / e4m3.quant_step_max(256.0)
    assert r == pytest.approx(8 / 7)
    assert round(r - 1, 2) == golden["dp_448_excess"]["value"]
    # between powers of two the step is larger (the sawtooth rises to 2^-3)
    for S in (3.0, 24.0, 192.0, 300.0, 384.0):
        assert e4m3.quant_step_max(S) > 1 / 16
    assert e4m3.quant_step_max(129.0) == pytest.approx(16.0 / 129.0)   # jumps to ~2^-3 just above 2^7


def test_normal_coverage(golden):
    S = golden["largest_safe_pow2_scale"]["value"]
    assert S == max(2 ** k for k in range(20) if 2 ** k <= golden["largest_safe_pow2_scale"]["max_finite"])
    assert e4m3.E4M3_MIN_NORMAL / S == golden["normal_coverage_S256"]["value"]

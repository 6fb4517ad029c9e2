"""Pins for the oracle's exact attention (O1) and P-cast block pipeline (O2).

What pins them:
* O1 against torch's scaled_dot_product_attention in fp64 on the CPU, an
  independent implementation (scale 1/sqrt(d), additive bias, causal mask,
  grouped kv heads);
* O2 with the cast switched off against O1: the online recurrence equals the
  two-pass softmax in exact arithmetic (FlashAttention blog, online-softmax
  section), for every order and block size, ragged last block included;
* special cases with a closed form: Q = 0 makes every p = 1 so O2 is the mean of
  the cast values (times 448/S once S saturates); a huge sink bias underflows
  every non-sink code so O2 with V = 1 is the sink mass written out by hand;
  one key block makes the two orders the same computation;
* the bf16 path against O1 within the 5e-3 acceptance bound;
* the two implementations (NumPy sequential / telescoped, C) against each other;
* planted mistakes (in the oracle, on the CPU) that these pins must catch.
"""
import math

import numpy as np
import pytest
import torch

import synthetic
from oracle import core, e4m3, reference


def _inputs(B, Hq, Hkv, N, d, seed):
    return synthetic.qkv_bf16(B, Hq, Hkv, N, d, seed)


def _sdpa_fp64(q_bits, k_bits, v_bits, bias, causal):
    q = torch.from_numpy(reference.bf16_to_f64(q_bits))
    k = torch.from_numpy(reference.bf16_to_f64(k_bits))
    v = torch.from_numpy(reference.bf16_to_f64(v_bits))
    N = q.shape[2]
    mask = torch.zeros(N, N, dtype=torch.float64)
    if bias is not None:
        mask = mask + torch.from_numpy(np.asarray(bias, dtype=np.float64))[None, :]
    if causal:
        mask = mask.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
    out = torch.nn.functional.scaled_dot_product_attention(
        q, k, v, attn_mask=mask, enable_gqa=q.shape[1] != k.shape[1])
    return out.numpy()


@pytest.mark.parametrize("causal", [False, True])
def test_exact_attention_matches_sdpa(causal):
    q, k, v = _inputs(2, 4, 2, 192, 64, 7)
    bias = synthetic.sink_bias(192, 5.0)
    ref = _sdpa_fp64(q, k, v, bias, causal)
    o1, _, _, _ = reference.attention_oracle(q, k, v, bias, causal, 256.0, 0, "kernel")
    assert np.max(np.abs(o1 - ref)) < 1e-12
    r = core.rows(q, k, v, bias, causal, 256.0, 0, "kernel")
    assert np.max(np.abs(r["o1"].reshape(ref.shape) - ref)) < 1e-12


@pytest.mark.parametrize("order", [0, 1])
@pytest.mark.parametrize("bc", [16, 64, 80])
@pytest.mark.parametrize("causal", [False, True])
def test_online_equals_full_softmax_without_cast(order, bc, causal):
    q, k, v = _inputs(1, 2, 1, 200, 32, 8)          # 200 keys: a ragged last block for every bc
    bias = synthetic.sink_bias(200, 9.0)
    o1, o2, _, _ = reference.attention_oracle(q, k, v, bias, causal, 256.0, order, "nocast", bc,
                                              sequential=True)
    assert np.max(np.abs(o2 - o1)) < 1e-12
    r = core.rows(q, k, v, bias, causal, 256.0, order, "nocast", bc=bc)
    assert np.max(np.abs(r["o2"].reshape(o1.shape) - o1)) < 1e-12


@pytest.mark.parametrize("mode", reference.MODES)
@pytest.mark.parametrize("order", [0, 1])
def test_twins_agree(mode, order):
    q, k, v = _inputs(1, 2, 2, 256, 64, 9)
    bias = synthetic.sink_bias(256, 7.0)
    for S in (1.0, 256.0, 448.0, 512.0):
        _, seq, ts, zs = reference.attention_oracle(q, k, v, bias, True, S, order, mode, sequential=True)
        _, vec, tv, zv = reference.attention_oracle(q, k, v, bias, True, S, order, mode)
        r = core.rows(q, k, v, bias, True, S, order, mode)
        assert np.max(np.abs(seq - vec)) < 1e-12
        assert np.max(np.abs(r["o2"].reshape(seq.shape) - seq)) < 1e-12
        assert np.array_equal(ts, tv) and np.array_equal(zs, zv)
        assert np.array_equal(r["total"].reshape(ts.shape), ts)
        assert np.array_equal(r["zero"].reshape(zs.shape), zs)


@pytest.mark.parametrize("mode", reference.MODES)
@pytest.mark.parametrize("order", [0, 1])
@pytest.mark.parametrize("causal", [False, True])
def test_twins_agree_with_a_partial_last_block(mode, order, causal):
    """N = 200: the last key block holds 8 keys; the C core, the sequential twin (which
    visits the keys of each block that exist) and the vectorised twin agree."""
    q, k, v = _inputs(1, 2, 1, 200, 64, 16)
    bias = synthetic.sink_bias(200, 7.0)
    for S in (1.0, 256.0, 512.0):
        _, seq, ts, zs = reference.attention_oracle(q, k, v, bias, causal, S, order, mode, sequential=True)
        _, vec, tv, zv = reference.attention_oracle(q, k, v, bias, causal, S, order, mode)
        r = core.rows(q, k, v, bias, causal, S, order, mode)
        assert np.max(np.abs(seq - vec)) < 1e-12
        assert np.max(np.abs(r["o2"].reshape(seq.shape) - seq)) < 1e-12
        assert np.array_equal(ts, tv) and np.array_equal(zs, zv)
        assert np.array_equal(r["total"].reshape(ts.shape), ts)
        assert np.array_equal(r["zero"].reshape(zs.shape), zs)


@pytest.mark.parametrize("S", [1.0, 2.0, 16.0, 256.0, 448.0])
@pytest.mark.parametrize("order", [0, 1])
def test_zero_queries_give_mean_of_cast_values(S, order):
    """Q = 0, no bias: every logit is 0, every p is 1, every code is E4M3(S) = S."""
    _, k, v = _inputs(1, 1, 1, 256, 64, 10)
    q = np.zeros_like(k)
    vh = e4m3.e4m3_rne(reference.bf16_to_f64(v[0, 0]))
    r = core.rows(q, k, v, None, False, S, order, "kernel")
    assert np.array_equal(r["o2"], np.broadcast_to(vh.mean(axis=0), r["o2"].shape)) or \
        np.max(np.abs(r["o2"] - vh.mean(axis=0))) < 1e-15
    # causal: row i averages keys 0..i
    rc = core.rows(q, k, v, None, True, S, order, "kernel")
    expect = np.cumsum(vh, axis=0) / np.arange(1, 257)[:, None]
    assert np.max(np.abs(rc["o2"] - expect)) < 1e-13


def test_zero_queries_saturate_above_448(golden):
    """S = 512 overflows E4M3: every code saturates to 448, so O2 = (448/512) mean(vhat)."""
    S = float(golden["scale_512_overflows"]["value"])
    _, k, v = _inputs(1, 1, 1, 128, 64, 11)
    q = np.zeros_like(k)
    vh = e4m3.e4m3_rne(reference.bf16_to_f64(v[0, 0]))
    r = core.rows(q, k, v, None, False, S, 0, "kernel")
    assert np.max(np.abs(r["o2"] - 0.875 * vh.mean(axis=0))) < 1e-15


def test_huge_sink_underflows_every_nonsink_and_keeps_it_in_the_sum():
    """Delta = 30, forward, S = 1, V = 1: non-sink p ~ e^-30 < 2^-10, all cast to 0.

    O2 = sum over the 4 sinks of E4M3(exp(s_j - m)) / sum over all keys of
    exp(s_j - m): the zeroed mass leaves the numerator but stays in the
    denominator (row sum from the un-cast P).
    """
    N, d = 128, 64
    q, k, _ = _inputs(1, 1, 1, N, d, 12)
    v = np.full_like(k, np.uint16(0x3F80))          # bf16 1.0
    bias = synthetic.sink_bias(N, 30.0)
    r = core.rows(q, k, v, bias, False, 1.0, 0, "kernel")
    s = (torch.from_numpy(reference.bf16_to_f64(q[0, 0])) @
         torch.from_numpy(reference.bf16_to_f64(k[0, 0])).T).numpy() / math.sqrt(d) + bias
    m = s.max(axis=1, keepdims=True)
    w = np.exp(s - m)
    expect = e4m3.e4m3_rne(w[:, :4]).sum(axis=1) / w.sum(axis=1)
    assert np.max(np.abs(r["o2"][:, 0] - expect)) < 1e-14
    assert np.all(r["zero"] == r["total"]) and np.all(r["total"] == N - 4)


@pytest.mark.parametrize("mode", ["kernel", "pages", "bf16"])
def test_single_block_orders_are_identical(mode):
    q, k, v = _inputs(1, 2, 2, 64, 128, 13)
    bias = synthetic.sink_bias(64, 7.0)
    for causal in (False, True):
        a = core.rows(q, k, v, bias, causal, 1.0, 0, mode)
        b = core.rows(q, k, v, bias, causal, 1.0, 1, mode)
        assert np.array_equal(a["o2"], b["o2"]) and np.array_equal(a["zero"], b["zero"])


def test_bf16_path_close_to_exact():
    """The no-cast bf16 path stays within 5e-3 of fp64 attention (Tiny shape)."""
    q, k, v = _inputs(1, 1, 1, 1024, 64, 1)
    bias = synthetic.sink_bias(1024, 7.0)
    r = core.rows(q, k, v, bias, False, 0.5, 0, "bf16")      # S is ignored in bf16 mode
    assert np.max(np.abs(r["o2"] - r["o1"])) < 5e-3


def test_slack_covers_eps_perturbed_codes():
    """Recomputing O2 with S*p perturbed by +/- eps/2 stays within the reported slack."""
    q, k, v = _inputs(1, 1, 1, 256, 64, 14)
    bias = synthetic.sink_bias(256, 7.0)
    eps = core.DEFAULT_EPS
    base = core.rows(q, k, v, bias, True, 1.0, 0, "kernel", eps=eps)
    for f in (1 - eps / 2, 1 + eps / 2):
        pert = core.rows(q, k, v, bias, True, f, 0, "kernel", eps=eps)   # S = f: S*p scaled by f
        dev = np.max(np.abs(pert["o2"] * f - base["o2"]), axis=1)         # undo the /S of the epilogue
        assert np.all(dev <= base["slack"] * 1.0001 + 1e-12)


# ---------------------------------------------------------------------------
# Planted mistakes: each must make one of the pins above fail.
# ---------------------------------------------------------------------------

def _fa1_local_max_emulator(s, v, S, order, mode, bc=64, nonsink=None):
    """The pipeline with P taken relative to the block's own max (FA1 pseudocode form)."""
    R, N = s.shape
    nonsink = np.ones(N, dtype=bool) if nonsink is None else nonsink
    tot = np.zeros(R, dtype=np.int64)
    zer = np.zeros(R, dtype=np.int64)
    for t in range((N + bc - 1) // bc):
        js = slice(t * bc, min((t + 1) * bc, N))
        blk = s[:, js]
        p = np.exp(blk - np.max(blk, axis=1, keepdims=True))
        c = e4m3.e4m3_rne(S * p)
        ns = np.isfinite(blk) & nonsink[js][None, :]
        tot += ns.sum(axis=1)
        zer += (ns & (c == 0)).sum(axis=1)
    return None, tot, zer


def test_planted_local_max_is_caught_by_collapse_rate():
    from oracle import theory
    rng = np.random.default_rng(5)
    s = rng.standard_normal((400, 1024))
    s[:, :4] += 7.0
    ns = np.ones(1024, dtype=bool)
    ns[:4] = False
    _, tot, zer = _fa1_local_max_emulator(s, None, 1.0, 0, "pages", 64, ns)
    assert abs(zer.sum() / tot.sum() - theory.f_exact(7.0, 1.0)) > 0.5   # the collapse disappears


def test_planted_cast_sum_is_caught_by_sink_case():
    """If the row sum were built from the cast P, V = 1 would give O2 = 1 exactly."""
    s = np.concatenate([[8.0], np.zeros(60)])[None, :]     # 60 keys at p = e^-8 < 2^-10
    v = np.ones((61, 1))
    c = e4m3.e4m3_rne(np.exp(s - s.max()))
    wrong = c.sum() / c.sum()
    right = reference.emulate_vectorized(s, v, 1.0, 0, "kernel")[0][0, 0]
    assert wrong == 1.0
    assert right == pytest.approx(1.0 / (1.0 + 60 * math.exp(-8.0)), rel=1e-14)


def test_planted_truncating_cast_is_caught_by_threshold():
    trunc = lambda x: np.floor(np.asarray(x) / 2.0 ** -9) * 2.0 ** -9   # noqa: E731
    assert trunc(3 * 2.0 ** -10) != e4m3.e4m3_rne(3 * 2.0 ** -10)
    assert e4m3.e4m3_rne(3 * 2.0 ** -10) == 2.0 ** -8


def test_planted_missing_scale_is_caught_by_sdpa():
    q, k, v = _inputs(1, 1, 1, 64, 64, 15)
    ref = _sdpa_fp64(q, k, v, None, False)
    qf, kf, vf = (reference.bf16_to_f64(x[0, 0]) for x in (q, k, v))
    s_wrong = qf @ kf.T                           # 1/sqrt(d) dropped
    assert np.max(np.abs(reference.exact_attention(s_wrong, vf) - ref[0, 0])) > 1e-3

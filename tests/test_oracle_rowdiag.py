"""Pins for oracle.rowdiag (per-row log-sum-exp and lost non-sink mass).

* lse against torch.logsumexp of the fp64 logits (a library routine);
* the zero decisions against the C core's underflow counter, row by row, over
  S, order, mask and bias (the core is pinned on its own in the other oracle tests);
* special cases: Delta = 30 forward S = 1 loses every non-sink key (lost = 1
  exactly); no sink and S = 256 loses nothing; rows with only sink keys give 0;
* the collapse model: on Gaussian Q, K (logits about N(0,1)) with four sinks at
  Delta = 7, forward order and S = 1, the mean lost mass over rows far from the
  sink block matches E[Phi(Delta + M_4 - 10 ln 2 - ln S - 1)] (the non-sink
  density weighted by exp(z) is the normal density shifted by one);
* a planted mistake (codes taken relative to the final max instead of the
  running max) changes the reverse-order result and fails.
"""
import numpy as np
import pytest

import synthetic
from oracle import core, e4m3, rowdiag, theory

torch = pytest.importorskip("torch")


def _logits(q_bits, k_bits, bias, causal):
    q = torch.from_numpy(((q_bits.astype(np.uint32)) << 16).view(np.float32).astype(np.float64))
    k = torch.from_numpy(((k_bits.astype(np.uint32)) << 16).view(np.float32).astype(np.float64))
    s = q @ k.transpose(-1, -2) / np.sqrt(q.shape[-1])
    if bias is not None:
        s = s + torch.from_numpy(bias.astype(np.float64))
    if causal:
        n = s.shape[-1]
        s = s.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), float("-inf"))
    return s


@pytest.mark.parametrize("N", [256, 200])
@pytest.mark.parametrize("causal", [False, True])
def test_lse_matches_torch(causal, N):
    q, k, _ = synthetic.qkv_bf16(1, 2, 2, N, 64, 61)
    bias = synthetic.random_bias(N, 61)
    r = rowdiag.rows(q, k, bias, causal, 256.0, 1)
    want = torch.logsumexp(_logits(q, k, bias, causal), dim=-1).numpy().ravel()
    assert np.max(np.abs(r["lse"] - want)) < 1e-12 * np.max(np.abs(want))


@pytest.mark.parametrize("S,order,causal,delta", [(1.0, 0, True, 7.0), (1.0, 1, True, 7.0),
                                                   (256.0, 0, False, 9.0), (448.0, 1, True, 12.0),
                                                   (3.0, 0, True, 5.0), (512.0, 0, True, 11.0)])
@pytest.mark.parametrize("N", [320, 300])  # 300: a partial last key block
def test_zero_decisions_match_core_counter(S, order, causal, delta, N):
    q, k, v = synthetic.qkv_bf16(1, 2, 2, N, 64, 62)
    bias = synthetic.sink_bias(N, delta)
    r = rowdiag.rows(q, k, bias, causal, S, order)
    c = core.rows(q, k, v, bias, causal, S, order, "kernel", want_exact=False)
    assert np.array_equal(r["zero"], c["zero"])
    assert r["zero"].sum() > 0


def test_strong_sink_loses_everything():
    q, k, _ = synthetic.qkv_bf16(1, 1, 1, 256, 64, 63)
    bias = synthetic.sink_bias(256, 30.0)
    r = rowdiag.rows(q, k, bias, True, 1.0, 0)
    assert np.all(r["lost"][:4] == 0.0)        # rows 0..3 see only sink keys
    assert np.all(r["lost"][4:] == 1.0)


def test_no_sink_loses_nothing():
    q, k, _ = synthetic.qkv_bf16(1, 2, 2, 256, 128, 64)
    r = rowdiag.rows(q, k, None, True, 256.0, 0)
    assert np.all(r["lost"] == 0.0) and np.all(r["zero"] == 0)


def test_lost_mass_matches_collapse_model():
    B, H, N, d = 1, 8, 4096, 128
    q, k, _ = synthetic.qkv_bf16(B, H, H, N, d, 2)
    bias = synthetic.sink_bias(N, 7.0)
    rng = np.random.default_rng(0)
    ids = np.sort(rng.choice(np.arange(H * N).reshape(H, N)[:, 1024:].ravel(), 2048, replace=False))
    r = rowdiag.rows(q, k, bias, True, 1.0, 0, ids)
    se = r["lost"].std() / np.sqrt(ids.size)
    model = theory.f_exact(7.0 - 1.0, 1.0)
    assert abs(r["lost"].mean() - model) < 4 * se + 0.01, (r["lost"].mean(), model, se)


def test_planted_final_max_is_caught():
    """Codes relative to the row's final max (not the running max) make reverse
    order behave like forward order: the reverse result then differs."""
    q, k, _ = synthetic.qkv_bf16(1, 1, 1, 1024, 64, 65)
    bias = synthetic.sink_bias(1024, 7.0)
    good = rowdiag.rows(q, k, bias, True, 1.0, 1)
    s = _logits(q, k, bias, True).numpy()[0, 0]
    m = np.max(s, axis=1, keepdims=True)
    with np.errstate(invalid="ignore"):
        w = np.where(np.isfinite(s), np.exp(s - m), 0.0)
    zero = np.isfinite(s) & (e4m3.e4m3_rne(w) == 0.0)
    ns = np.isfinite(s) & (bias == 0)[None, :]
    tot = np.sum(np.where(ns, w, 0.0), axis=1)
    wrong = np.where(tot > 0, np.sum(np.where(ns & zero, w, 0.0), axis=1) / np.where(tot > 0, tot, 1), 0)
    assert np.mean(wrong) > np.mean(good["lost"]) + 0.3

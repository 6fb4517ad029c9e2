"""Pins for oracle.backward (gradients by recomputation from lse, cast passed through).

* with the exact forward's O and lse, dQ, dK, dV equal torch autograd of
  softmax(Q K^T / sqrt(d) + bias) V in fp64, with causal masks and grouped kv heads;
* the rows of dS sum to zero when O is exact (D_i = sum_j P_ij dP_ij);
* finite differences of a scalar loss agree with the analytic gradient;
* a planted mistake (D_i dropped) fails the autograd pin.
"""
import math

import numpy as np
import pytest

import synthetic
from oracle import backward

torch = pytest.importorskip("torch")


def _f64(bits):
    return torch.from_numpy(((bits.astype(np.uint32)) << 16).view(np.float32).astype(np.float64))


def _autograd(qb, kb, vb, dob, bias, causal):
    q, k, v = (_f64(x).requires_grad_(True) for x in (qb, kb, vb))
    G = q.shape[1] // k.shape[1]
    kk, vv = k.repeat_interleave(G, dim=1), v.repeat_interleave(G, dim=1)
    s = q @ kk.transpose(-1, -2) / math.sqrt(q.shape[-1])
    if bias is not None:
        s = s + torch.from_numpy(bias.astype(np.float64))
    if causal:
        n = s.shape[-1]
        s = s.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), float("-inf"))
    o = torch.softmax(s, dim=-1) @ vv
    o.backward(_f64(dob))
    return q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (4, 2)])
def test_matches_autograd(causal, Hq, Hkv):
    qb, kb, vb = synthetic.qkv_bf16(1, Hq, Hkv, 96, 32, 101)
    dob = synthetic.gaussian_bf16(101, 3, qb.shape)
    bias = synthetic.sink_bias(96, 3.0)
    o, lse = backward.forward_exact(qb, kb, vb, bias, causal)
    dq, dk, dv = backward.grads(qb, kb, vb, o, dob, lse, bias, causal)
    aq, ak, av = _autograd(qb, kb, vb, dob, bias, causal)
    for x, y in ((dq, aq), (dk, ak), (dv, av)):
        assert np.max(np.abs(x - y)) <= 1e-10 * max(1.0, np.max(np.abs(y)))


def test_ds_rows_sum_to_zero():
    qb, kb, vb = synthetic.qkv_bf16(1, 1, 1, 64, 32, 102)
    dob = synthetic.gaussian_bf16(102, 3, qb.shape)
    o, lse = backward.forward_exact(qb, kb, vb, None, True)
    # dQ = dS K / sqrt(d): with K = all-ones rows, dQ_i = (sum_j dS_ij) / sqrt(d) * 1
    ones = np.full(kb.shape, 0x3F80, dtype=np.uint16)                 # bf16 1.0
    o1, lse1 = backward.forward_exact(qb, ones, vb, None, True)
    dq, _, _ = backward.grads(qb, ones, vb, o1, dob, lse1, None, True)
    assert np.max(np.abs(dq)) < 1e-12


def test_finite_differences():
    qb, kb, vb = synthetic.qkv_bf16(1, 1, 1, 32, 16, 103)
    dob = synthetic.gaussian_bf16(103, 3, qb.shape)
    bias = synthetic.sink_bias(32, 2.0)
    q, k, v, do = (backward._bf16(x) for x in (qb, kb, vb, dob))

    def loss(qq, kk, vv):
        s = qq[0, 0] @ kk[0, 0].T / 4.0 + bias
        s = np.where(np.tril(np.ones((32, 32), dtype=bool)), s, -np.inf)
        w = np.exp(s - s.max(axis=1, keepdims=True))
        return float(np.sum((w / w.sum(axis=1, keepdims=True)) @ vv[0, 0] * do[0, 0]))

    o, lse = backward.forward_exact(qb, kb, vb, bias, True)
    dq, dk, dv = backward.grads(qb, kb, vb, o, dob, lse, bias, True)
    rng = np.random.default_rng(0)
    h = 1e-6
    for arr, g in ((q, dq), (k, dk), (v, dv)):
        for _ in range(5):
            i, c = int(rng.integers(32)), int(rng.integers(16))
            a, bb = arr.copy(), arr.copy()
            a[0, 0, i, c] += h
            bb[0, 0, i, c] -= h
            args_a = [a if arr is x else x for x in (q, k, v)]
            args_b = [bb if arr is x else x for x in (q, k, v)]
            fd = (loss(*args_a) - loss(*args_b)) / (2 * h)
            assert abs(fd - g[0, 0, i, c]) < 1e-6 * max(1.0, abs(fd))


def test_planted_missing_d_is_caught():
    qb, kb, vb = synthetic.qkv_bf16(1, 1, 1, 64, 32, 104)
    dob = synthetic.gaussian_bf16(104, 3, qb.shape)
    o, lse = backward.forward_exact(qb, kb, vb, None, False)
    _, _, _ = backward.grads(qb, kb, vb, o, dob, lse, None, False)
    # D = 0 is what the formulas give for O = 0
    dq0, _, _ = backward.grads(qb, kb, vb, np.zeros_like(o), dob, lse, None, False)
    aq, _, _ = _autograd(qb, kb, vb, dob, None, False)
    assert np.max(np.abs(dq0 - aq)) > 1e-3


def test_sampled_equals_full():
    qb, kb, vb = synthetic.qkv_bf16(1, 4, 2, 128, 32, 105)
    dob = synthetic.gaussian_bf16(105, 3, qb.shape)
    bias = synthetic.sink_bias(128, 4.0)
    o, lse = backward.forward_exact(qb, kb, vb, bias, True)
    dq, dk, dv, bnd = backward.grads(qb, kb, vb, o, dob, lse, bias, True, with_bounds=True)
    rows = [(0, 0, 0), (0, 3, 127), (0, 2, 64)]
    keys = [(0, 0, 0), (0, 1, 127), (0, 1, 5)]
    sq, sk, sv, sb = backward.grads_sampled(qb, kb, vb, o, dob, lse, bias, True, rows, keys)
    for n, (b, h, i) in enumerate(rows):
        assert np.allclose(sq[n], dq[b, h, i], rtol=1e-10, atol=1e-12)
        assert np.allclose(sb["dq"][n], bnd["dq"][b, h, i], rtol=1e-10, atol=1e-12)
        assert np.allclose(sb["dq2"][n], bnd["dq2"][b, h, i], rtol=1e-10, atol=1e-12)
    for n, (b, g, j) in enumerate(keys):
        assert np.allclose(sk[n], dk[b, g, j], rtol=1e-10, atol=1e-12)
        assert np.allclose(sv[n], dv[b, g, j], rtol=1e-10, atol=1e-12)
        assert np.allclose(sb["dk"][n], bnd["dk"][b, g, j], rtol=1e-10, atol=1e-12)
        assert np.allclose(sb["dk2"][n], bnd["dk2"][b, g, j], rtol=1e-10, atol=1e-12)
        assert np.allclose(sb["dv"][n], bnd["dv"][b, g, j], rtol=1e-10, atol=1e-12)

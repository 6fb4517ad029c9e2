"""Pins for oracle.decode (decode rows, keys in ranges that each run the P-cast
pipeline, merged by the online-softmax rescale).

* one range is the P-cast path itself: equal to the C core (pinned on its own)
  run causally with the decode rows placed at the last positions of the
  sequence -- outputs, pair counts and zero counts, with grouped kv heads and a
  sink bias, both orders, several S;
* without the cast the merge is exact attention for every range size and order
  (the online-softmax recurrence, FlashAttention blog "La ricorrenza softmax
  online");
* the running max is local to a range: with S = 256 and a strong sink, forward
  order zeroes non-sink codes only in the range holding the sink; with one range
  it zeroes them everywhere;
* a planted mistake (merging without rescaling to the common max) fails.
"""
import numpy as np
import pytest

import synthetic
from oracle import core, decode


def _inputs(B, Hq, Hkv, Nq, Nk, d, seed):
    q = synthetic.gaussian_bf16(seed, 0, (B, Hq, Nq, d))
    k = synthetic.gaussian_bf16(seed, 1, (B, Hkv, Nk, d))
    v = synthetic.gaussian_bf16(seed, 2, (B, Hkv, Nk, d))
    return q, k, v


@pytest.mark.parametrize("Nk", [320, 300, 258])  # 300, 258: a partial last key block (258: 2 keys)
@pytest.mark.parametrize("S,order,Nq", [(1.0, 0, 1), (256.0, 1, 1), (448.0, 0, 3), (3.0, 1, 4)])
def test_one_range_is_the_pcast_path(S, order, Nq, Nk):
    B, Hq, Hkv, d = 2, 4, 2, 64
    q, k, v = _inputs(B, Hq, Hkv, Nq, Nk, d, 81)
    bias = synthetic.sink_bias(Nk, 7.0)
    r = decode.rows(q, k, v, bias, S, order, split_keys=-(-Nk // 64) * 64)  # one range
    qf = np.zeros((B, Hq, Nk, d), dtype=np.uint16)
    qf[:, :, Nk - Nq:] = q
    ids = np.array([(b * Hq + h) * Nk + Nk - Nq + i for b in range(B) for h in range(Hq) for i in range(Nq)])
    c = core.rows(qf, k, v, bias, True, S, order, "kernel", row_ids=ids)
    o2 = r["o2"].reshape(-1, d)
    assert np.max(np.abs(o2 - c["o2"])) < 1e-12
    assert np.max(np.abs(r["o1"].reshape(-1, d) - c["o1"])) < 1e-12
    assert np.array_equal(r["total"].ravel(), c["total"]) and np.array_equal(r["zero"].ravel(), c["zero"])


@pytest.mark.parametrize("Nk", [1024, 1000])
@pytest.mark.parametrize("split", [64, 128, 192, 1024])
@pytest.mark.parametrize("order", [0, 1])
def test_nocast_merge_is_exact(split, order, Nk):
    q, k, v = _inputs(1, 2, 1, 2, Nk, 32, 82)
    bias = synthetic.sink_bias(Nk, 5.0)
    r = decode.rows(q, k, v, bias, 1.0, order, split, mode="nocast")
    assert np.max(np.abs(r["o2"] - r["o1"])) < 1e-12


def test_running_max_is_local_to_a_range():
    Nk, split = 1024, 256
    q, k, v = _inputs(1, 2, 2, 1, Nk, 64, 83)
    bias = synthetic.sink_bias(Nk, 25.0)
    one = decode.rows(q, k, v, bias, 256.0, 0, split_keys=Nk)
    many = decode.rows(q, k, v, bias, 256.0, 0, split_keys=split)
    # one range: every non-sink key sits far below the sink max
    assert np.all(one["zero"] == one["total"])
    # ranges: only the range with the sink (keys 0..255, 252 non-sink) loses its keys
    assert np.all(many["zero"] == split - 4)
    assert np.all(many["total"] == Nk - 4)


def test_planted_merge_without_rescale_is_caught():
    q, k, v = _inputs(1, 1, 1, 1, 512, 32, 84)
    bias = synthetic.sink_bias(512, 7.0)
    r = decode.rows(q, k, v, bias, 1.0, 0, 128, mode="nocast")
    # the same ranges merged by plain sums of (l, A) without the e^(m_r - M) factors
    kf = decode._bf16(k[0, 0])
    vf = decode._bf16(v[0, 0])
    s = kf @ decode._bf16(q[0, 0, 0]) / np.sqrt(32) + bias
    num, den = np.zeros(32), 0.0
    for r0 in range(0, 512, 128):
        m = s[r0:r0 + 128].max()
        p = np.exp(s[r0:r0 + 128] - m)
        num += p @ vf[r0:r0 + 128]
        den += p.sum()
    assert np.max(np.abs(num / den - r["o1"][0, 0, 0])) > 1e-3

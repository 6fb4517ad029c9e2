"""GPU parity of the FP8-logit decode (attn_decode_pcast_qk8) against oracle.decode
on the dequantised Q and K of oracle.qk8 (one power-of-two scale per query row and
per 64-key block of each head).

Tolerance per row, as for the FP8-logit forward: the FP8 matrix cores accumulate
the code products with a relative error below ACC_REL of the sum of their
magnitudes, so with Delta = ACC_REL log2(e)/sqrt(d) max_j sum_d |q_d k_jd| (log2
units, over the dequantised operands) every p, the running max weights and l move
by a relative delta = 2 ln2 Delta at most.  Codes then agree except within a
relative delta of a rounding point (the oracle's slack, taken with eps = max delta
+ 2^-14), and the rest moves O by at most 3.5 delta A, A the oracle's output with
|V|.  Per row: max-abs <= 1e-3 + slack + 3.5 delta A; relative MSE against exact
attention of the dequantised inputs within 5 % of the oracle's; per (b, h) pair
counts equal and zero counts within the near-threshold pairs.
"""
import numpy as np
import pytest

import synthetic
from oracle import decode, qk8
from tests import _parity

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sna():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import softmax_numerics_amd
    softmax_numerics_amd.load_library()
    return softmax_numerics_amd


def _run(sna, qb, kb, vb, bias, S, order, split, stats=True):
    B, Hq, Nq, d = qb.shape
    Hkv, Nk = kb.shape[1], kb.shape[2]
    q, k, v = (_parity.to_gpu_bf16(x) for x in (qb, kb, vb))
    st = torch.cuda.current_stream().cuda_stream
    ws8 = torch.empty(sna.workspace_bytes_qk8(B, Hkv, Nk, d), dtype=torch.uint8, device="cuda")
    assert sna.prepare_qk8(k.data_ptr(), v.data_ptr(), B, Hkv, Nk, d, ws8.data_ptr(), st) == 0
    ws = torch.empty(sna.decode_workspace_bytes(B, Hkv, Nk, d, split), dtype=torch.uint8, device="cuda")
    out = torch.full((B, Hq, Nq, d), float("nan"), device="cuda")
    sts = torch.full((sna.stats_words(B, Hq, Nq),), -1, dtype=torch.int64, device="cuda") if stats else None
    bt = None if bias is None else torch.from_numpy(bias).cuda()
    rc = sna.attn_decode_pcast_qk8(q.data_ptr(), ws8.data_ptr(), 0 if bt is None else bt.data_ptr(),
                                   B, Hq, Hkv, Nq, Nk, d, S, order, split, out.data_ptr(),
                                   0 if sts is None else sts.data_ptr(), ws.data_ptr(), st)
    assert rc == 0, sna.strerror(rc)
    torch.cuda.synchronize()
    return out.cpu().numpy(), (None if sts is None else sts.cpu().numpy().reshape(B, Hq, 2))


def _logit_delta(qd, kd, Nk):
    """Per decode row: 2 ln2 Delta, Delta the logit error bound over the keys it sees."""
    q = _parity._bf16_f64(qd)
    k = _parity._bf16_f64(kd)
    B, Hq, Nq, d = q.shape
    grp = Hq // k.shape[1]
    out = np.empty((B, Hq, Nq))
    for b in range(B):
        for h in range(Hq):
            mags = np.abs(q[b, h]) @ np.abs(k[b, h // grp]).T  # [Nq, Nk]
            for i in range(Nq):
                out[b, h, i] = np.max(mags[i, :Nk - Nq + i + 1])
    return 2.0 * np.log(2.0) * _parity.ACC_REL * _parity.LOG2E / np.sqrt(d) * out


def _case(sna, name, B, Hq, Hkv, Nq, Nk, d, bias, S, order, split, seed, sub=None):
    print(f"\n[case] decode qk8 {name}: B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} S={S} order={order} "
          f"split={split} seed={seed} compared={sub}", flush=True)
    qb, kb, vb = synthetic.decode_qkv_bf16(B, Hq, Hkv, Nq, Nk, d, seed)
    out, st = _run(sna, qb, kb, vb, bias, S, order, split)
    if sub is not None:
        nb, nkv = sub
        nq = nkv * (Hq // Hkv)
        qb, kb, vb, out, st = qb[:nb, :nq], kb[:nb, :nkv], vb[:nb, :nkv], out[:nb, :nq], st[:nb, :nq]
    qd, _ = qk8.quantize_q(qb)
    kd, _ = qk8.quantize_k(kb)
    delta = _logit_delta(qd, kd, Nk)
    ref = decode.rows(qd, kd, vb, bias, S, order, split, eps=float(delta.max()) + _parity.EPS)
    abs_v = np.asarray(vb, dtype=np.uint16) & np.uint16(0x7FFF)
    a_row = np.max(np.abs(decode.rows(qd, kd, abs_v, bias, S, order, split)["o2"]), axis=-1)
    d_ = out.shape[-1]
    got = out.reshape(-1, d_).astype(np.float64)
    o2, o1 = ref["o2"].reshape(-1, d_), ref["o1"].reshape(-1, d_)
    dev = np.max(np.abs(got - o2), axis=1)
    tol = _parity.ATOL + ref["slack"].ravel() + 3.5 * delta.ravel() * a_row.ravel()
    assert np.all(dev <= tol), f"worst dev {dev.max():.3g}, ratio {np.max(dev / tol):.3g}"
    e1 = np.sum(o1 ** 2)
    rel_gpu, rel_o2 = np.sum((got - o1) ** 2) / e1, np.sum((o2 - o1) ** 2) / e1
    assert abs(rel_gpu - rel_o2) <= 0.05 * rel_o2 + 1e-15, f"relMSE {rel_gpu:.4g} vs {rel_o2:.4g}"
    tot, zer, amb = (ref[k].sum(axis=2) for k in ("total", "zero", "zero_amb"))
    assert np.array_equal(st[..., 0], tot), "pair counts differ"
    assert np.all(np.abs(st[..., 1] - zer) <= amb), "zero counts differ beyond near ties"
    rep = {"max_dev": float(dev.max()), "worst_ratio": float(np.max(dev / tol)), "relmse_gpu": float(rel_gpu),
           "relmse_oracle": float(rel_o2), "logit_delta_max": float(delta.max())}
    print(f"[case] decode qk8 {name}: {rep}", flush=True)
    return rep


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("order", [0, 1])
@pytest.mark.parametrize("S", [1.0, 256.0, 448.0])
@pytest.mark.parametrize("split", [64, 1024])
def test_grid(sna, d, order, S, split):
    # GQA groups of 4, one row each; ranges of one block and of all 16
    _case(sna, "grid", 2, 8, 2, 1, 1024, d, synthetic.sink_bias(1024, 7.0), S, order, split, 191)


@pytest.mark.parametrize("Hq,Hkv,Nq", [(32, 8, 8), (4, 1, 3)])
def test_rows_and_groups(sna, Hq, Hkv, Nq):
    _case(sna, f"rows G={Hq // Hkv} Nq={Nq}", 1, Hq, Hkv, Nq, 640, 128, synthetic.sink_bias(640, 7.0), 256.0,
          1, 256, 192)


@pytest.mark.parametrize("Nk", [1000, 1025])
@pytest.mark.parametrize("order", [0, 1])
def test_ragged_cache(sna, Nk, order):
    # a partial last key block: its codes padded with zeros, its scale from the keys that exist
    _case(sna, f"ragged Nk={Nk}", 2, 4, 1, 6, Nk, 128, synthetic.sink_bias(Nk, 7.0), 256.0, order, 1024, 194)


@pytest.mark.parametrize("bias_kind", ["none", "random"])
def test_bias_kinds(sna, bias_kind):
    bias = None if bias_kind == "none" else synthetic.random_bias(768, 193)
    _case(sna, f"bias {bias_kind}", 1, 4, 2, 2, 768, 128, bias, 256.0, 0, 256, 193)


def test_decode_full_size(sna):
    w = synthetic.DECODE_WORKLOADS["decode"]
    delta, S, order = w.cases[0]
    _case(sna, w.name, w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, synthetic.sink_bias(w.Nk, delta), S, order,
          w.split_keys, w.seed, sub=(2, 2))


def test_deterministic(sna):
    qb, kb, vb = synthetic.decode_qkv_bf16(2, 8, 2, 4, 2048, 128, 196)
    bias = synthetic.sink_bias(2048, 7.0)
    a, sa = _run(sna, qb, kb, vb, bias, 256.0, 1, 512)
    b, sb = _run(sna, qb, kb, vb, bias, 256.0, 1, 512)
    c, _ = _run(sna, qb, kb, vb, bias, 256.0, 1, 512, stats=False)
    assert np.array_equal(a, b) and np.array_equal(sa, sb) and np.array_equal(a, c)

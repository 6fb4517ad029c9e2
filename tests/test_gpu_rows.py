"""GPU tests of attn_fwd_pcast_rows (per-row log-sum-exp and lost non-sink mass).

* out and stats equal attn_fwd_pcast_prepared's bit for bit (the diagnostics take
  the kernel's sequential step for every block, which computes the same numbers);
  with lost NULL the pipelined kernel writes lse alone, bit-identical to the lse
  written beside the lost mass;
* lse and lost against oracle.rowdiag: |lse_gpu - lse| <= 1e-4 + 1e-5 |lse|
  (fp32 logits, exp2 and log2: about 1e-6 relative each); |lost_gpu - lost| <=
  2e-5 + 1e-4 lost + lost_amb, lost_amb the oracle's share of non-sink mass whose
  zero decision sits within a relative 2^-14 of the threshold (the counters'
  near-tie rule);
* the full-size Throughput rows at Delta = 7, forward, S = 1: the measured lost
  mass next to the collapse model's prediction.
"""
import numpy as np
import pytest

import synthetic
from oracle import rowdiag
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


def _run(sna, qb, kb, vb, bias, causal, S, order):
    B, Hq, N, d = qb.shape
    Hkv = kb.shape[1]
    q, k, v = (_parity.to_gpu_bf16(x) for x in (qb, kb, vb))
    bt = None if bias is None else torch.from_numpy(bias).cuda()
    ws = torch.empty(sna.workspace_bytes(B, Hkv, N, d, S), dtype=torch.uint8, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    assert sna.prepare_v(v.data_ptr(), B, Hkv, N, d, S, ws.data_ptr(), st) == 0
    res = {}
    for name, rows in (("plain", False), ("rows", True), ("lse_only", True)):
        out = torch.full((B, Hq, N, d), float("nan"), device="cuda")
        stats = torch.full((sna.stats_words(B, Hq, N),), -1, dtype=torch.int64, device="cuda")
        bp = 0 if bt is None else bt.data_ptr()
        if rows:
            lse = torch.full((B, Hq, N), float("nan"), device="cuda")
            lost = torch.full((B, Hq, N), float("nan"), device="cuda")
            # lost NULL: the pipelined kernel writes lse alone
            lost_ptr = 0 if name == "lse_only" else lost.data_ptr()
            rc = sna.attn_fwd_pcast_rows(q.data_ptr(), k.data_ptr(), ws.data_ptr(), bp, B, Hq, Hkv, N, d,
                                         causal, S, order, out.data_ptr(), stats.data_ptr(), lse.data_ptr(),
                                         lost_ptr, st)
        else:
            rc = sna.attn_fwd_pcast_prepared(q.data_ptr(), k.data_ptr(), ws.data_ptr(), bp, B, Hq, Hkv, N, d,
                                             causal, S, order, out.data_ptr(), stats.data_ptr(), st)
        assert rc == 0, sna.strerror(rc)
        torch.cuda.synchronize()
        res[name] = (out.cpu().numpy(), stats.cpu().numpy())
        if name == "rows":
            res["lse"], res["lost"] = lse.cpu().numpy().ravel(), lost.cpu().numpy().ravel()
        elif name == "lse_only":
            res["lse_only_lse"] = lse.cpu().numpy().ravel()
            assert torch.isnan(lost).all().item(), "lost written although not requested"
    return res


def _check(res, qb, kb, bias, causal, S, order, ids=None):
    a, sa = res["plain"]
    b, sb = res["rows"]
    assert np.array_equal(a, b) and np.array_equal(sa, sb), "diagnostics changed out or stats"
    c, sc = res["lse_only"]
    assert np.array_equal(a, c) and np.array_equal(sa, sc), "lse alone changed out or stats"
    assert np.array_equal(res["lse_only_lse"], res["lse"]), "lse alone differs from lse with the lost mass"
    r = rowdiag.rows(qb, kb, bias, causal, S, order, ids)
    sel = slice(None) if ids is None else ids
    lse, lost = res["lse"][sel], res["lost"][sel]
    dl = np.abs(lse - r["lse"])
    assert np.all(dl <= 1e-4 + 1e-5 * np.abs(r["lse"])), f"lse off by {dl.max():.3g}"
    dm = np.abs(lost - r["lost"])
    assert np.all(dm <= 2e-5 + 1e-4 * r["lost"] + r["lost_amb"]), f"lost off by {dm.max():.3g}"
    return {"lse_dev": float(dl.max()), "lost_dev": float(dm.max()), "lost_mean_gpu": float(lost.mean()),
            "lost_mean_oracle": float(r["lost"].mean())}


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("order", [0, 1])
@pytest.mark.parametrize("S", [1.0, 256.0, 448.0])
def test_small_grid(sna, d, causal, order, S):
    print(f"\n[case] rows grid d={d} causal={causal} order={order} S={S}", flush=True)
    qb, kb, vb = synthetic.qkv_bf16(2, 4, 2, 320, d, 71)
    bias = synthetic.sink_bias(320, 7.0)
    rep = _check(_run(sna, qb, kb, vb, bias, causal, S, order), qb, kb, bias, causal, S, order)
    print(f"[case] rows grid: {rep}", flush=True)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("order", [0, 1])
def test_ragged_sequence(sna, causal, order):
    print(f"\n[case] rows ragged N=200 causal={causal} order={order}", flush=True)
    qb, kb, vb = synthetic.qkv_bf16(1, 2, 1, 200, 128, 73)
    bias = synthetic.sink_bias(200, 7.0)
    rep = _check(_run(sna, qb, kb, vb, bias, causal, 1.0, order), qb, kb, bias, causal, 1.0, order)
    print(f"[case] rows ragged: {rep}", flush=True)


@pytest.mark.parametrize("bias_kind", ["none", "random", "strong"])
def test_bias_kinds(sna, bias_kind):
    print(f"\n[case] rows bias {bias_kind}", flush=True)
    N = 384
    qb, kb, vb = synthetic.qkv_bf16(1, 3, 3, N, 128, 72)
    bias = {"none": None, "random": synthetic.random_bias(N, 72), "strong": synthetic.sink_bias(N, 30.0)}[bias_kind]
    res = _run(sna, qb, kb, vb, bias, True, 1.0, 0)
    rep = _check(res, qb, kb, bias, True, 1.0, 0)
    if bias_kind == "strong":
        lost = res["lost"].reshape(3, N)
        assert np.all(lost[:, :4] == 0.0) and np.all(lost[:, 4:] == 1.0)
    print(f"[case] rows bias: {rep}", flush=True)


def test_throughput_lost_mass(sna):
    w = synthetic.WORKLOADS["throughput"]
    print(f"\n[case] rows throughput forward S=1 delta=7", flush=True)
    qb, kb, vb = synthetic.qkv_bf16(w.B, w.Hq, w.Hkv, w.N, w.d, w.seed)
    bias = synthetic.sink_bias(w.N, 7.0)
    res = _run(sna, qb, kb, vb, bias, w.causal, 1.0, 0)
    ids = _parity.block_rows(w.B, w.Hq, w.N, _parity.sample_blocks(w.B, w.Hq, w.N, 8, w.seed))
    rep = _check(res, qb, kb, bias, w.causal, 1.0, 0, ids)
    model = sna.lost_mass_model(7.0, 1.0)
    far = res["lost"].reshape(w.B * w.Hq, w.N)[:, 1024:]
    rep["lost_mean_all_rows_from_1024"] = float(far.mean())
    rep["model"] = model
    print(f"[case] rows throughput: {rep}", flush=True)
    assert abs(far.mean() - model) < 0.02


def test_zero_scale_is_rejected(sna):
    q = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16, device="cuda")
    out = torch.empty(1, 1, 64, 64, device="cuda")
    ws = torch.empty(sna.workspace_bytes(1, 1, 64, 64, 0.0), dtype=torch.uint8, device="cuda")
    rc = sna.attn_fwd_pcast_rows(q.data_ptr(), q.data_ptr(), ws.data_ptr(), 0, 1, 1, 1, 64, 64, 1, 0.0, 0,
                                 out.data_ptr(), 0, out.data_ptr(), 0, 0)
    assert rc == sna.PCAST_ENOTSUP

"""The P-cast pages' error trends, reproduced by the GPU kernel (kernel mode: V in
E4M3 as the FP8 P.V needs) on the Sweep shape: B=1, H=8, N=4096, d=128, causal,
Q/K/V i.i.d. N(0,1) in bf16, sink bias Delta on keys 0..3.  MSE is the mean over
all output elements of (O_gpu - O_exact)^2 with O_exact the oracle's fp64
attention.

Checked: at Delta = 7 forward S = 1 is the worst of {forward, reverse} x
{1, 256} and of S = 448 forward; S = 256 beats S = 448 forward; reverse adds
nothing once S = 256; S = 512 saturates; the forward S = 1 underflow fraction
crosses 1/2 between Delta = 5 and 6 and matches the collapse model; the gain of
reverse S = 256 over forward S = 1 grows with N.  In kernel mode V's own E4M3
rounding adds the same error to every configuration, so the ratios are smaller
than the pages' (the oracle's kernel mode gives 1.18 at N = 4096); the
directions are what is asserted.
"""
import numpy as np
import pytest

import synthetic
from oracle import core
from tests import _parity

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

N, D, H = 4096, 128, 8


@pytest.fixture(scope="module")
def sna():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import softmax_numerics_amd
    softmax_numerics_amd.load_library()
    return softmax_numerics_amd


@pytest.fixture(scope="module")
def sweep(sna):
    q, k, v = synthetic.qkv_bf16(1, H, H, N, D, 2)
    gq, gk, gv = (_parity.to_gpu_bf16(x) for x in (q, k, v))
    exact = {}
    cache = {}

    def run(delta, S, order, n=N, heads=H):
        key = (delta, S, order, n, heads)
        if key in cache:
            return cache[key]
        qq, kk, vv = (t[:, :heads, :n] for t in (gq, gk, gv))
        qq, kk, vv = qq.contiguous(), kk.contiguous(), vv.contiguous()
        bias = synthetic.sink_bias(n, delta)
        out, st = sna.forward(qq, kk, vv, torch.from_numpy(bias).cuda(), causal=True, S=S, order=order, stats=True)
        torch.cuda.synchronize()
        if (delta, n, heads) not in exact:
            print(f"\n[case] trends: exact attention delta={delta} N={n} H={heads}", flush=True)
            ex = core.rows(q[:, :heads, :n].copy(), k[:, :heads, :n].copy(), v[:, :heads, :n].copy(), bias, True,
                           256.0, 1, "kernel", want_exact=True)["o1"]
            exact[(delta, n, heads)] = ex
        o1 = exact[(delta, n, heads)]
        got = out.double().cpu().numpy().reshape(-1, D)
        s = st.cpu().numpy()
        r = {"mse": float(np.mean((got - o1) ** 2)), "underflow": float(s[..., 1].sum() / s[..., 0].sum())}
        print(f"[case] trends: delta={delta} S={S} order={order} N={n} H={heads}: {r}", flush=True)
        cache[key] = r
        return r
    return run


def test_forward_s1_is_worst(sweep):
    base = sweep(7.0, 1.0, "forward")["mse"]
    for S, order in ((1.0, "reverse"), (256.0, "forward"), (256.0, "reverse"), (448.0, "forward")):
        assert base / sweep(7.0, S, order)["mse"] > 1.1


def test_s256_beats_s448_forward(sweep):
    assert sweep(7.0, 256.0, "forward")["mse"] < sweep(7.0, 448.0, "forward")["mse"]


def test_reverse_adds_nothing_at_s256(sweep):
    a, b = sweep(7.0, 256.0, "forward")["mse"], sweep(7.0, 256.0, "reverse")["mse"]
    assert abs(a - b) / a < 0.02


def test_s512_saturates(sweep):
    assert sweep(7.0, 512.0, "forward")["mse"] > 5 * sweep(7.0, 256.0, "forward")["mse"]


def test_collapse_crosses_half_and_matches_model(sna, sweep):
    f5, f6, f7 = (sweep(d, 1.0, "forward")["underflow"] for d in (5.0, 6.0, 7.0))
    assert f5 < 0.5 < f6
    assert abs(f7 - sna.underflow_model(7.0, 1.0)) < 0.03


def test_gain_grows_with_n(sweep):
    ratios = [sweep(7.0, 1.0, "forward", n=n, heads=2)["mse"] / sweep(7.0, 256.0, "reverse", n=n, heads=2)["mse"]
              for n in (1024, 2048, 4096)]
    print(f"[case] trends: fwd S=1 / rev S=256 at N=1024, 2048, 4096: {ratios}", flush=True)
    assert ratios[0] < ratios[1] < ratios[2]


@pytest.mark.parametrize("name", ["gqa", "long"])
def test_gain_at_scale(sna, name):
    """The forward-S=1 / reverse-S=256 MSE ratio at the GQA (N = 65536) and Long
    (N = 131072) shapes, on 256 rows sampled uniformly over heads and positions: the
    GPU's MSE against fp64 attention agrees with the oracle's kernel-mode MSE on the
    same rows (within 3 %), and the ratio exceeds the Sweep shape's (1.18 at N = 4096).
    In the oracle's pages mode (V exact) the same ratio is about 2 at N = 4096, 3.3
    at 16k, 5.9 at 64k and 11 at 128k (Delta = 7)."""
    w = synthetic.WORKLOADS[name]
    print(f"\n[case] trends at scale: {name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N}", flush=True)
    qb, kb, vb = synthetic.qkv_bf16(w.B, w.Hq, w.Hkv, w.N, w.d, w.seed)
    q, k, v = (_parity.to_gpu_bf16(x) for x in (qb, kb, vb))
    rng = np.random.default_rng(5)
    ids = np.sort(rng.choice(w.B * w.Hq * w.N, 256, replace=False))
    bias = synthetic.sink_bias(w.N, 7.0)
    bt = torch.from_numpy(bias).cuda()
    idx = torch.from_numpy(ids).cuda()
    mse = {}
    for S, order in ((1.0, "forward"), (256.0, "reverse")):
        out, _ = sna.forward(q, k, v, bt, causal=True, S=S, order=order)
        got = out.view(-1, w.d)[idx].double().cpu().numpy()
        del out
        torch.cuda.synchronize()
        r = core.rows(qb, kb, vb, bias, True, S, 0 if order == "forward" else 1, "kernel", row_ids=ids)
        mse[S] = (float(np.mean((got - r["o1"]) ** 2)), float(np.mean((r["o2"] - r["o1"]) ** 2)))
        print(f"[case] trends at scale: {name} S={S} {order}: MSE gpu {mse[S][0]:.4e} oracle {mse[S][1]:.4e}",
              flush=True)
        assert abs(mse[S][0] - mse[S][1]) <= 0.03 * mse[S][1]
    ratio = mse[1.0][0] / mse[256.0][0]
    print(f"[case] trends at scale: {name}: fwd S=1 / rev S=256 = {ratio:.2f}", flush=True)
    assert ratio > 1.3

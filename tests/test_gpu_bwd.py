"""GPU parity of the backward (attn_bwd_pcast) against oracle.backward.

The forward runs on the GPU first (attn_fwd_pcast_rows: its O and lse are the
backward's inputs, and the oracle is given the same O and lse).  Tolerance per
element, from the GPU's arithmetic:
* P (for dV) and dS (for dQ, dK) are rounded to bf16 (8 significant bits, RNE:
  a relative 2^-8 each): 2^-7 M with M the oracle's sum of magnitudes
  (|dS| |K| / sqrt(d), |dS|^T |Q| / sqrt(d), |P|^T |dO|), twice the bound;
* dP and D are fp32 sums of 128 products, so dP - D carries an absolute error of
  about 2^-17 of the magnitudes it is summed from; where it nearly cancels (rows
  dominated by a sink) that is not small against dS: 2^-15 M2, M2 =
  P (|dO||V|^T + |dO||O|) |K| / sqrt(d) (and its transpose with |Q| for dK);
* exp2 and the fp32 logits move P by about 1e-6 relative: inside the first term.
"""
import numpy as np
import pytest

import synthetic
from oracle import backward
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


def _run(sna, qb, kb, vb, dob, bias, causal, S=256.0, order=1):
    B, Hq, N, d = qb.shape
    Hkv = kb.shape[1]
    q, k, v, do = (_parity.to_gpu_bf16(x) for x in (qb, kb, vb, dob))
    bt = None if bias is None else torch.from_numpy(bias).cuda()
    bp = 0 if bt is None else bt.data_ptr()
    st = torch.cuda.current_stream().cuda_stream
    ws = torch.empty(sna.workspace_bytes(B, Hkv, N, d, S), dtype=torch.uint8, device="cuda")
    o = torch.empty((B, Hq, N, d), device="cuda")
    lse = torch.empty((B, Hq, N), device="cuda")
    assert sna.prepare_v(v.data_ptr(), B, Hkv, N, d, S, ws.data_ptr(), st) == 0
    rc = sna.attn_fwd_pcast_rows(q.data_ptr(), k.data_ptr(), ws.data_ptr(), bp, B, Hq, Hkv, N, d, causal, S,
                                 order, o.data_ptr(), 0, lse.data_ptr(), 0, st)
    assert rc == 0, sna.strerror(rc)
    dq = torch.full((B, Hq, N, d), float("nan"), device="cuda")
    dk = torch.full((B, Hkv, N, d), float("nan"), device="cuda")
    dv = torch.full((B, Hkv, N, d), float("nan"), device="cuda")
    wb = torch.empty(sna.bwd_workspace_bytes(B, Hq, Hkv, N, d), dtype=torch.uint8, device="cuda")
    rc = sna.attn_bwd_pcast(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                            bp, B, Hq, Hkv, N, d, causal, dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                            wb.data_ptr(), st)
    assert rc == 0, sna.strerror(rc)
    torch.cuda.synchronize()
    return (o.cpu().numpy(), lse.cpu().numpy(), dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy())


def _check(name, got, want, bound, bound2=None):
    tol = 2.0 ** -7 * bound + 1e-7
    if bound2 is not None:
        tol = tol + 2.0 ** -15 * bound2
    dev = np.abs(got - want)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    assert np.all(dev <= tol), f"{name}: worst {dev.max():.3g}, ratio {np.max(dev / tol):.3g}"
    return float(np.max(dev / tol))


def _case(sna, name, B, Hq, Hkv, N, d, causal, bias, seed):
    print(f"\n[case] bwd {name}: B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} causal={causal} seed={seed}", flush=True)
    qb, kb, vb = synthetic.qkv_bf16(B, Hq, Hkv, N, d, seed)
    dob = synthetic.gaussian_bf16(seed, 3, qb.shape)
    o, lse, dq, dk, dv = _run(sna, qb, kb, vb, dob, bias, causal)
    rq, rk, rv, bnd = backward.grads(qb, kb, vb, o, dob, lse, bias, causal, with_bounds=True)
    rep = {"dq": _check("dQ", dq, rq, bnd["dq"], bnd["dq2"]), "dk": _check("dK", dk, rk, bnd["dk"], bnd["dk2"]),
           "dv": _check("dV", dv, rv, bnd["dv"])}
    print(f"[case] bwd {name}: worst deviation / tolerance {rep}", flush=True)
    return rep


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_small(sna, d, causal):
    # N = 320: partial 128-row / 128-key workgroups; grouped kv heads; sink bias
    _case(sna, "small", 2, 4, 2, 320, d, causal, synthetic.sink_bias(320, 7.0), 111)


@pytest.mark.parametrize("B,Hq,Hkv,N,d,causal", [
    (2, 4, 1, 64, 64, True),      # one key block: most waves of both kernels idle
    (1, 8, 1, 192, 64, False),    # eight query heads per kv head, a partial 256-row block
    (1, 2, 2, 448, 128, True),    # seven key blocks, diagonal blocks at both parities
    (1, 16, 2, 384, 128, False),  # the dK/dV walk over eight query heads
])
def test_shapes(sna, B, Hq, Hkv, N, d, causal):
    _case(sna, "shape", B, Hq, Hkv, N, d, causal, synthetic.sink_bias(N, 7.0), 116 + N + d)


@pytest.mark.parametrize("bias_kind", ["none", "random"])
def test_bias_kinds(sna, bias_kind):
    bias = None if bias_kind == "none" else synthetic.random_bias(256, 112)
    _case(sna, f"bias {bias_kind}", 1, 3, 3, 256, 128, True, bias, 112)


def test_mid_size(sna):
    _case(sna, "mid", 1, 8, 2, 2048, 128, True, synthetic.sink_bias(2048, 7.0), 113)


def test_throughput_sampled(sna):
    w = synthetic.WORKLOADS["throughput"]
    print("\n[case] bwd throughput sampled rows and keys", flush=True)
    qb, kb, vb = synthetic.qkv_bf16(w.B, w.Hq, w.Hkv, w.N, w.d, w.seed)
    dob = synthetic.gaussian_bf16(w.seed, 3, qb.shape)
    bias = synthetic.sink_bias(w.N, 7.0)
    o, lse, dq, dk, dv = _run(sna, qb, kb, vb, dob, bias, w.causal)
    rng = np.random.default_rng(114)
    rows = [(int(rng.integers(w.B)), int(rng.integers(w.Hq)), int(rng.integers(w.N))) for _ in range(24)]
    rows += [(0, 0, 0), (w.B - 1, w.Hq - 1, w.N - 1)]
    keys = [(int(rng.integers(w.B)), int(rng.integers(w.Hkv)), int(rng.integers(w.N))) for _ in range(24)]
    keys += [(0, 0, 0), (w.B - 1, w.Hkv - 1, w.N - 1)]
    rq, rk, rv, bnd = backward.grads_sampled(qb, kb, vb, o, dob, lse, bias, w.causal, rows, keys)
    gq = np.array([dq[b, h, i] for b, h, i in rows])
    gk = np.array([dk[b, g, j] for b, g, j in keys])
    gv = np.array([dv[b, g, j] for b, g, j in keys])
    rep = {"dq": _check("dQ", gq, rq, bnd["dq"], bnd["dq2"]), "dk": _check("dK", gk, rk, bnd["dk"], bnd["dk2"]),
           "dv": _check("dV", gv, rv, bnd["dv"])}
    print(f"[case] bwd throughput: worst deviation / tolerance {rep}", flush=True)


def test_deterministic(sna):
    qb, kb, vb = synthetic.qkv_bf16(1, 4, 2, 512, 128, 115)
    dob = synthetic.gaussian_bf16(115, 3, qb.shape)
    a = _run(sna, qb, kb, vb, dob, None, True)
    b = _run(sna, qb, kb, vb, dob, None, True)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("N", [100, 200])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("bias_kind", ["none", "sink"])
def test_ragged_sequence(sna, N, causal, bias_kind):
    # N not a multiple of 64: the backward runs on whole-block copies (zero rows, bias -inf past N)
    bias = None if bias_kind == "none" else synthetic.sink_bias(N, 7.0)
    _case(sna, f"ragged N={N} bias={bias_kind}", 2, 4, 2, N, 64 if N == 100 else 128, causal, bias, 117 + N)


@pytest.mark.parametrize("N", [256, 150])
@pytest.mark.parametrize("bias_kind", ["none", "sink"])
def test_autograd_attention_equals_direct_calls(sna, bias_kind, N):
    """softmax_numerics_amd.attention under autograd: out equals the plain forward and the
    gradients equal the C backward's (rounded to bf16) on the same dO, bit for bit."""
    B, Hq, Hkv, d, seed = 1, 4, 2, 64, 91
    print(f"\n[case] autograd attention: bias={bias_kind}", flush=True)
    qb, kb, vb = synthetic.qkv_bf16(B, Hq, Hkv, N, d, seed)
    q, k, v = (_parity.to_gpu_bf16(x).requires_grad_(True) for x in (qb, kb, vb))
    bias = None if bias_kind == "none" else torch.from_numpy(synthetic.sink_bias(N, 7.0)).cuda()
    out = sna.attention(q, k, v, bias, causal=True, S=256.0, order="reverse")
    g = torch.from_numpy(np.random.default_rng(seed).standard_normal((B, Hq, N, d)).astype(np.float32)).cuda()
    out.backward(g)
    torch.cuda.synchronize()
    ref, _ = sna.forward(q.detach(), k.detach(), v.detach(), bias, causal=True, S=256.0, order="reverse")
    assert torch.equal(out.detach(), ref)
    st = torch.cuda.current_stream().cuda_stream
    ws = torch.empty(sna.workspace_bytes(B, Hkv, N, d, 256.0), dtype=torch.uint8, device="cuda")
    o = torch.empty((B, Hq, N, d), device="cuda")
    lse = torch.empty((B, Hq, N), device="cuda")
    bp = 0 if bias is None else bias.data_ptr()
    assert sna.prepare_v(v.data_ptr(), B, Hkv, N, d, 256.0, ws.data_ptr(), st) == 0
    assert sna.attn_fwd_pcast_rows(q.data_ptr(), k.data_ptr(), ws.data_ptr(), bp, B, Hq, Hkv, N, d, True, 256.0, 1,
                                   o.data_ptr(), 0, lse.data_ptr(), 0, st) == 0
    do = g.to(torch.bfloat16).contiguous()
    dq = torch.empty((B, Hq, N, d), device="cuda")
    dk = torch.empty((B, Hkv, N, d), device="cuda")
    dv = torch.empty_like(dk)
    wb = torch.empty(sna.bwd_workspace_bytes(B, Hq, Hkv, N, d), dtype=torch.uint8, device="cuda")
    assert sna.attn_bwd_pcast(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                              bp, B, Hq, Hkv, N, d, True, dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                              wb.data_ptr(), st) == 0
    torch.cuda.synchronize()
    for got, want in ((q.grad, dq), (k.grad, dk), (v.grad, dv)):
        assert got.dtype == torch.bfloat16 and torch.equal(got, want.to(torch.bfloat16))


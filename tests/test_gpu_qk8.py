"""GPU parity of the FP8-logit path (attn_fwd_pcast_qk8) against the oracle.

The K pre-pass is compared bit for bit with the oracle's quantisation
(oracle.qk8): the exponent of every 64-key block and the E4M3 code of every
element.  Q is rounded inside the attention kernel, row by row: feeding the
kernel the oracle's rounded Q (and K) instead of the originals must give the
same output bit for bit.  The attention output is compared with the oracle run
on the dequantised Q and K, within the tolerance tests/_parity.compare_qk8
derives from the FP8 matrix cores' accumulation error.
"""
import numpy as np
import pytest

import synthetic
from oracle import core, e4m3, qk8
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


def _up(x):
    return (x + 255) // 256 * 256


def _prepare(sna, kb, vb):
    B, Hkv, N, d = kb.shape
    k, v = (_parity.to_gpu_bf16(x) for x in (kb, vb))
    ws = torch.zeros(sna.workspace_bytes_qk8(B, Hkv, N, d), dtype=torch.uint8, device="cuda")
    rc = sna.prepare_qk8(k.data_ptr(), v.data_ptr(), B, Hkv, N, d, ws.data_ptr(),
                         torch.cuda.current_stream().cuda_stream)
    assert rc == sna.PCAST_OK, sna.strerror(rc)
    torch.cuda.synchronize()
    w = ws.cpu().numpy()
    nb = -(-N // 64)  # whole key blocks: a partial last block is padded
    nkv = B * Hkv * nb * 64 * d
    off_k = _up(nkv)
    off_e = _up(off_k + nkv)
    k8 = w[off_k:off_k + nkv].reshape(B, Hkv, nb * 64, d)
    assert not np.any(k8[:, :, N:]), "codes of the padding rows"
    return {"k8": k8[:, :, :N],
            "kexp": w[off_e:off_e + 4 * B * Hkv * nb].view(np.int32).reshape(B, Hkv, nb)}


def _check_k_prepass(parts, bits):
    x = ((bits.astype(np.uint32) & 0xFFFF) << 16).view(np.float32).astype(np.float64)
    _, exps = qk8.quantize_k(bits)
    assert np.array_equal(parts["kexp"], exps), "key block exponents"
    B, H, N, d = bits.shape
    e = np.repeat(exps, 64, axis=2)[:, :, :N, None]
    want = e4m3.e4m3_encode(np.ldexp(x, -e))
    got = parts["k8"]
    assert not np.any((got & 0x7F) == 0x7F), "NaN code"
    # equal values (+0 and -0 are both zero to the matrix cores)
    assert np.array_equal(e4m3.DECODE_TABLE[got], e4m3.DECODE_TABLE[want]), "K codes"


def _scaled_heads(B, H, N, d, seed, tensor_id):
    """Gaussian heads at very different scales, with a zero head, an outlier
    channel and a head whose max sits exactly on 448 * 2^k."""
    bits = synthetic.gaussian_bf16(seed, tensor_id, (B, H, N, d))
    x = ((bits.astype(np.uint32)) << 16).view(np.float32).reshape(B * H, N, d).copy()
    scales = [1.0, 2.0 ** -20, 3.0e4, 0.0, 1.0, 7.5e-3, 1.0, 2.0 ** 40]
    for i in range(B * H):
        x[i] *= np.float32(scales[i % len(scales)])
    if B * H > 4:
        x[4, :, 5] *= 200.0                    # one outlier channel
    if B * H > 6:
        x[6] = np.clip(x[6], -3.0, 3.0)
        x[6, min(3, N - 1), 7] = 448.0 * 2.0 ** -7  # amax exactly 448 * 2^-7 (= 3.5)
    u = x.reshape(B, H, N, d).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)   # back to bf16, RNE


def test_k_prepass_bit_exact(sna):
    print("\n[case] qk8 K pre-pass: B=2 Hkv=4 N=192 d=128", flush=True)
    kb = _scaled_heads(2, 4, 192, 128, 41, 1)
    vb = synthetic.gaussian_bf16(41, 2, kb.shape)
    _check_k_prepass(_prepare(sna, kb, vb), kb)


def test_k_prepass_bit_exact_d64(sna):
    print("\n[case] qk8 K pre-pass: B=1 Hkv=8 N=640 d=64", flush=True)
    kb = _scaled_heads(1, 8, 640, 64, 42, 1)
    # blocks inside one head at very different scales too
    x = ((kb.astype(np.uint32)) << 16).view(np.float32).copy()
    x[0, 0, 64:128] *= np.float32(2.0 ** 30)
    x[0, 0, 128:192] = 0.0
    x[0, 0, 200, 3] = np.float32(448.0 * 2.0 ** 3)
    kb = (x.view(np.uint32) >> 16).astype(np.uint16)
    vb = synthetic.gaussian_bf16(42, 2, kb.shape)
    _check_k_prepass(_prepare(sna, kb, vb), kb)


def test_v_copy_matches_plain_prepass(sna):
    """The fused pre-pass writes the same V operand copy as pcast_prepare_v."""
    print("\n[case] qk8 V copy: B=2 Hkv=2 N=256 d=128", flush=True)
    kb = synthetic.gaussian_bf16(48, 1, (2, 2, 256, 128))
    vb = synthetic.gaussian_bf16(48, 2, (2, 2, 256, 128))
    k, v = (_parity.to_gpu_bf16(x) for x in (kb, vb))
    ws8 = torch.zeros(sna.workspace_bytes_qk8(2, 2, 256, 128), dtype=torch.uint8, device="cuda")
    ws = torch.zeros(sna.workspace_bytes(2, 2, 256, 128, 256.0), dtype=torch.uint8, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    assert sna.prepare_qk8(k.data_ptr(), v.data_ptr(), 2, 2, 256, 128, ws8.data_ptr(), st) == 0
    assert sna.prepare_v(v.data_ptr(), 2, 2, 256, 128, 256.0, ws.data_ptr(), st) == 0
    torch.cuda.synchronize()
    assert torch.equal(ws8[:ws.numel()].cpu(), ws.cpu())


def _run_qk8(sna, qb, kb, vb, bias, causal, S, order, stats=True):
    q, k, v = (_parity.to_gpu_bf16(x) for x in (qb, kb, vb))
    bt = None if bias is None else torch.from_numpy(bias).cuda()
    out, st = sna.forward(q, k, v, bt, causal=causal, S=S, order=order, stats=stats, qk_fp8=True)
    torch.cuda.synchronize()
    return out.cpu().numpy(), (None if st is None else st.cpu().numpy())


def _run(sna, qb, kb, vb, bias, causal, S, order):
    """The P-cast forward with bf16 logits, for comparison."""
    q, k, v = (_parity.to_gpu_bf16(x) for x in (qb, kb, vb))
    bt = None if bias is None else torch.from_numpy(bias).cuda()
    out, st = sna.forward(q, k, v, bt, causal=causal, S=S, order=order, stats=True)
    torch.cuda.synchronize()
    return out.cpu().numpy(), st.cpu().numpy()


def _case(sna, name, B, Hq, Hkv, N, d, causal, bias, S, order, seed, blocks=None, qkv=None):
    print(f"\n[case] qk8 {name}: B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} causal={causal} S={S} "
          f"order={order} seed={seed}", flush=True)
    qb, kb, vb = synthetic.qkv_bf16(B, Hq, Hkv, N, d, seed) if qkv is None else qkv
    out, st = _run_qk8(sna, qb, kb, vb, bias, causal, S, order)
    qd, _ = qk8.quantize_q(qb)
    kd, _ = qk8.quantize_k(kb)
    if isinstance(blocks, int):
        blocks = _parity.sample_blocks(B, Hq, N, blocks, seed)
    rep = _parity.compare_qk8(out, st, qd, kd, vb, bias, causal, S, order, blocks)
    print(f"[case] qk8 {name}: {rep}", flush=True)
    return rep


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("order", [0, 1])
@pytest.mark.parametrize("S", [1.0, 256.0, 448.0, 512.0])
def test_small_grid(sna, d, causal, order, S):
    # five key blocks, a half-empty last row block, grouped kv heads, sink bias 7
    _case(sna, "grid", 2, 4, 2, 320, d, causal, synthetic.sink_bias(320, 7.0), S, order, 43)


def test_k_prepass_bit_exact_partial_block(sna):
    # N = 200: the last key block holds 8 keys, its scale from their max (the padding is 0)
    print("\n[case] qk8 K pre-pass: B=2 Hkv=4 N=200 d=128", flush=True)
    kb = _scaled_heads(2, 4, 200, 128, 45, 1)
    vb = synthetic.gaussian_bf16(45, 2, kb.shape)
    _check_k_prepass(_prepare(sna, kb, vb), kb)


@pytest.mark.parametrize("N", [100, 200])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("S,order", [(256.0, 1), (1.0, 0)])
def test_ragged_sequence(sna, N, causal, S, order):
    _case(sna, f"ragged N={N}", 2, 4, 2, N, 64 if N == 100 else 128, causal, synthetic.sink_bias(N, 7.0), S, order,
          46 + N)


@pytest.mark.parametrize("order", [0, 1])
def test_random_bias(sna, order):
    _case(sna, "random bias", 1, 3, 3, 384, 128, True, synthetic.random_bias(384, 44), 256.0, order, 44)


def test_scaled_heads(sna):
    # heads at scales from 2^-20 to 2^40 and a zero head: the row and block
    # exponents must cancel exactly in the logits
    B, Hq, Hkv, N, d = 1, 8, 8, 256, 128
    qb = _scaled_heads(B, Hq, N, d, 45, 0)
    kb = np.ascontiguousarray(_scaled_heads(B, Hkv, N, d, 45, 1)[:, ::-1])
    vb = synthetic.gaussian_bf16(45, 2, kb.shape)
    # keep the logits moderate: a power of two per Q head brings max|q| max|k| near 30
    qf = ((qb.astype(np.uint32)) << 16).view(np.float32)
    kf = ((kb.astype(np.uint32)) << 16).view(np.float32)
    for h in range(Hq):
        aq = np.max(np.abs(qf[0, h])) or 1.0
        ak = np.max(np.abs(kf[0, h])) or 1.0
        qf[0, h] *= np.float32(2.0 ** np.round(np.log2(30.0 / aq / ak)))
    qb = (qf.view(np.uint32) >> 16).astype(np.uint16)
    _case(sna, "scaled heads", B, Hq, Hkv, N, d, True, None, 256.0, 1, 45, qkv=(qb, kb, vb))


@pytest.mark.parametrize("d", [64, 128])
def test_rounded_inputs_give_the_same_output(sna, d):
    """Q and K replaced by the oracle's rounded values: the kernel's own rounding
    of Q (per row) and the pre-pass's of K (per block) are then identities up to
    a power of two, so the output is the same bit for bit."""
    print(f"\n[case] qk8 rounded inputs, d={d}", flush=True)
    qb, kb, vb = synthetic.qkv_bf16(2, 4, 2, 320, d, 49)
    x = ((qb.astype(np.uint32)) << 16).view(np.float32).copy()
    x[:, :, ::5] *= np.float32(2.0 ** -9)            # rows at different scales
    qb = (x.view(np.uint32) >> 16).astype(np.uint16)
    qd, _ = qk8.quantize_q(qb)
    kd, _ = qk8.quantize_k(kb)
    bias = synthetic.sink_bias(320, 7.0)
    a, sa = _run_qk8(sna, qb, kb, vb, bias, True, 256.0, 1)
    b, sb = _run_qk8(sna, qd, kd, vb, bias, True, 256.0, 1)
    assert np.array_equal(a, b) and np.array_equal(sa, sb)


def test_single_block_orders_identical(sna):
    print("\n[case] qk8 one key block, both orders", flush=True)
    qb, kb, vb = synthetic.qkv_bf16(2, 2, 2, 64, 128, 46)
    bias = synthetic.sink_bias(64, 7.0)
    a, sa = _run_qk8(sna, qb, kb, vb, bias, True, 256.0, 0)
    b, sb = _run_qk8(sna, qb, kb, vb, bias, True, 256.0, 1)
    assert np.array_equal(a, b) and np.array_equal(sa, sb)


def test_deterministic(sna):
    print("\n[case] qk8 determinism", flush=True)
    qb, kb, vb = synthetic.qkv_bf16(1, 4, 4, 1024, 128, 47)
    bias = synthetic.sink_bias(1024, 7.0)
    a, sa = _run_qk8(sna, qb, kb, vb, bias, True, 256.0, 1)
    b, sb = _run_qk8(sna, qb, kb, vb, bias, True, 256.0, 1)
    c, _ = _run_qk8(sna, qb, kb, vb, bias, True, 256.0, 1, stats=False)
    assert np.array_equal(a, b) and np.array_equal(sa, sb) and np.array_equal(a, c)


def test_zero_scale_is_rejected(sna):
    q = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sna.PcastError) as ei:
        sna.forward(q, q, q, None, S=0.0, qk_fp8=True)
    assert ei.value.code == sna.PCAST_ENOTSUP


W = synthetic.WORKLOADS


@pytest.mark.parametrize("S,order", [(256.0, 1), (1.0, 0)])
def test_throughput_full_size(sna, S, order):
    w = W["throughput"]
    _case(sna, "throughput", w.B, w.Hq, w.Hkv, w.N, w.d, w.causal, synthetic.sink_bias(w.N, 7.0), S, order,
          w.seed, blocks=8)


def test_gqa_full_size(sna):
    w = W["gqa"]
    _case(sna, "gqa", w.B, w.Hq, w.Hkv, w.N, w.d, w.causal, synthetic.sink_bias(w.N, 7.0), 256.0, 1,
          w.seed, blocks=6)


# ---- FP8 logits with the random Hadamard rotation ----

def _signs(d, seed):
    return np.random.default_rng(seed).choice(np.array([-1, 1], dtype=np.int8), size=d)


def _prepare_rot(sna, qb, kb, vb, signs):
    B, Hq, N, d = qb.shape
    Hkv = kb.shape[1]
    q, k, v = (_parity.to_gpu_bf16(x) for x in (qb, kb, vb))
    sg = torch.from_numpy(signs).cuda()
    ws = torch.zeros(sna.workspace_bytes_qk8_rot(B, Hq, Hkv, N, d), dtype=torch.uint8, device="cuda")
    rc = sna.prepare_qk8_rot(q.data_ptr(), k.data_ptr(), v.data_ptr(), sg.data_ptr(), B, Hq, Hkv, N, d,
                             ws.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == sna.PCAST_OK, sna.strerror(rc)
    torch.cuda.synchronize()
    return ws


def _rot_run(sna, qb, kb, vb, bias, causal, S, order, signs):
    B, Hq, N, d = qb.shape
    Hkv = kb.shape[1]
    ws = _prepare_rot(sna, qb, kb, vb, signs)
    out = torch.empty((B, Hq, N, d), device="cuda")
    st = torch.empty(sna.stats_words(B, Hq, N), dtype=torch.int64, device="cuda")
    bt = None if bias is None else torch.from_numpy(bias).cuda()
    rc = sna.attn_fwd_pcast_qk8_rot_prepared(ws.data_ptr(), 0 if bt is None else bt.data_ptr(), B, Hq, Hkv, N, d,
                                             causal, S, order, out.data_ptr(), st.data_ptr(),
                                             torch.cuda.current_stream().cuda_stream)
    assert rc == sna.PCAST_OK, sna.strerror(rc)
    torch.cuda.synchronize()
    return out.cpu().numpy(), st.cpu().numpy().reshape(B, Hq, -1, 2)


@pytest.mark.parametrize("d,N", [(64, 192), (128, 192), (128, 200), (64, 37), (128, 1)])
def test_rotation_prepass_bit_exact(sna, d, N):
    print(f"\n[case] qk8 rotation pre-pass d={d} N={N}", flush=True)
    B, Hq, Hkv = 2, 4, 2
    nb = -(-N // 64)
    qb = _scaled_heads(B, Hq, N, d, 51, 0)
    kb = _scaled_heads(B, Hkv, N, d, 51, 1)
    vb = synthetic.gaussian_bf16(51, 2, kb.shape)
    signs = _signs(d, 51)
    w = _prepare_rot(sna, qb, kb, vb, signs).cpu().numpy()
    nkv, nq = B * Hkv * nb * 64 * d, B * Hq * N * d  # K codes in whole key blocks, Q codes per row
    off_k = _up(nkv)
    off_ke = _up(off_k + nkv)
    off_q = _up(off_ke + 4 * B * Hkv * nb)
    off_qe = _up(off_q + nq)
    k8 = w[off_k:off_k + nkv].reshape(B, Hkv, nb * 64, d)
    ke = w[off_ke:off_ke + 4 * B * Hkv * nb].view(np.int32).reshape(B, Hkv, nb)
    q8 = w[off_q:off_q + nq].reshape(qb.shape)
    qe = w[off_qe:off_qe + 4 * B * Hq * N].view(np.int32).reshape(B, Hq, N)
    # rows past the sequence are zeros (of either sign: a sign flip makes -0, code 0x80)
    assert not e4m3.DECODE_TABLE[k8[:, :, N:]].any(), "K rows past the sequence"
    sg = signs.astype(np.float64)
    for codes, exps, bits, rows in ((q8, qe, qb, 1), (k8[:, :, :N], ke, kb, 64)):
        x = qk8.rotate(bits, sg)
        _, want_e = qk8.quantize_values(x, rows)
        assert np.array_equal(exps, want_e), "exponents"
        e = np.repeat(want_e, rows, axis=2)[:, :, :N, None]
        want = e4m3.e4m3_encode(np.ldexp(x, -e))
        assert np.array_equal(e4m3.DECODE_TABLE[codes], e4m3.DECODE_TABLE[want]), "codes"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("S,order", [(256.0, 1), (1.0, 0)])
def test_rotation_parity(sna, d, causal, S, order):
    print(f"\n[case] qk8 rotation parity d={d} causal={causal} S={S} order={order}", flush=True)
    qb, kb, vb = synthetic.qkv_bf16(2, 4, 2, 320, d, 52)
    bias = synthetic.sink_bias(320, 7.0)
    signs = _signs(d, 52)
    out, st = _rot_run(sna, qb, kb, vb, bias, causal, S, order, signs)
    qd, kd, _, _ = qk8.quantize_rotated(qb, kb, signs.astype(np.float64))
    rep = _parity.compare_qk8(out, st, qd, kd, vb, bias, causal, S, order)
    print(f"[case] qk8 rotation parity: {rep}", flush=True)


@pytest.mark.parametrize("N", [1, 100, 200])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("S,order", [(256.0, 1), (1.0, 0)])
def test_rotation_parity_ragged(sna, N, causal, S, order):
    d = 64 if N == 100 else 128
    print(f"\n[case] qk8 rotation parity ragged N={N} d={d} causal={causal} S={S} order={order}", flush=True)
    qb, kb, vb = synthetic.qkv_bf16(2, 4, 2, N, d, 54)
    bias = synthetic.sink_bias(N, 7.0)
    signs = _signs(d, 54)
    out, st = _rot_run(sna, qb, kb, vb, bias, causal, S, order, signs)
    qd, kd, _, _ = qk8.quantize_rotated(qb, kb, signs.astype(np.float64))
    rep = _parity.compare_qk8(out, st, qd, kd, vb, bias, causal, S, order)
    print(f"[case] qk8 rotation parity ragged: {rep}", flush=True)


def _outlier_inputs(B, Hq, Hkv, N, d, seed, mult):
    qb, kb, vb = synthetic.qkv_bf16(B, Hq, Hkv, N, d, seed)
    chans = [3, 40, 77, 100][: 4 if d == 128 else 2]
    out = []
    for bits in (qb, kb):
        x = ((bits.astype(np.uint32)) << 16).view(np.float32).copy()
        x[..., chans] *= np.float32(mult)
        u = x.view(np.uint32).astype(np.uint64)
        out.append(((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16))
    return out[0], out[1], vb


def test_rotation_helps_with_outlier_channels(sna):
    """Four channels of Q and K 30x larger (with the scale of Q lowered so the logits
    stay moderate): the output error against exact attention of the unrounded inputs
    drops with the rotation."""
    B, Hq, Hkv, N, d = 1, 4, 4, 1024, 128
    qb, kb, vb = _outlier_inputs(B, Hq, Hkv, N, d, 53, 30.0)
    x = ((qb.astype(np.uint32)) << 16).view(np.float32) * np.float32(2.0 ** -5)
    qb = (x.view(np.uint32) >> 16).astype(np.uint16)
    bias = synthetic.sink_bias(N, 7.0)
    print("\n[case] qk8 rotation with outlier channels", flush=True)
    plain, _ = _run_qk8(sna, qb, kb, vb, bias, True, 256.0, 1)
    rot, _ = _rot_run(sna, qb, kb, vb, bias, True, 256.0, 1, _signs(d, 53))
    base, _ = _run(sna, qb, kb, vb, bias, True, 256.0, 1)
    ex = core.rows(qb, kb, vb, bias, True, 256.0, 1, "kernel", want_exact=True)["o1"]
    mse = {name: float(np.mean((o.reshape(-1, d) - ex) ** 2)) for name, o in
           (("bf16 logits", base), ("fp8 logits", plain), ("fp8 logits rotated", rot))}
    print(f"[case] qk8 rotation with outliers: MSE {mse}, plain / rotated {mse['fp8 logits'] / mse['fp8 logits rotated']:.2f}",
          flush=True)
    assert mse["fp8 logits rotated"] < mse["fp8 logits"]

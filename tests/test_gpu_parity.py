"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every case prints its name before touching the GPU.  Small shapes compare
every row; the full-size workloads compare whole 64-row blocks sampled across
heads and positions (the first and last blocks always included), in the same
launch configuration the benchmark times.
"""
import numpy as np
import pytest

import synthetic
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


def _run(sna, qb, kb, vb, bias, causal, S, order, stats=True):
    q, k, v = (_parity.to_gpu_bf16(x) for x in (qb, kb, vb))
    bt = None if bias is None else torch.from_numpy(bias).cuda()
    out, st = sna.forward(q, k, v, bt, causal=causal, S=S, order=order, stats=stats)
    torch.cuda.synchronize()
    return out.cpu().numpy(), (None if st is None else st.cpu().numpy())


def _case(sna, name, B, Hq, Hkv, N, d, causal, delta, S, order, seed, blocks=None):
    print(f"\n[case] {name}: B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} causal={causal} delta={delta} "
          f"S={S} order={order} seed={seed}", flush=True)
    qb, kb, vb = synthetic.qkv_bf16(B, Hq, Hkv, N, d, seed)
    bias = None if delta is None else synthetic.sink_bias(N, delta)
    out, st = _run(sna, qb, kb, vb, bias, causal, S, order)
    if isinstance(blocks, int):
        blocks = _parity.sample_blocks(B, Hq, N, blocks, seed)
    rep = _parity.compare(out, st, qb, kb, vb, bias, causal, S, order, blocks)
    print(f"[case] {name}: {rep}", flush=True)
    return rep


@pytest.mark.parametrize("S", [1.0, 256.0, 448.0, 0.0])
def test_tiny(sna, S):
    _case(sna, "tiny", 1, 1, 1, 1024, 64, False, 7.0, S, 0, 1)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("order", [0, 1])
@pytest.mark.parametrize("S", [1.0, 2.0, 256.0, 448.0, 512.0, 3.0, 0.0])
def test_small_grid(sna, d, causal, order, S):
    # N = 320: five key blocks and a half-empty last row block; grouped kv heads
    _case(sna, "grid", 2, 4, 2, 320, d, causal, 7.0, S, order, 21)


@pytest.mark.parametrize("delta", [None, 0.0, 3.0, 30.0])
@pytest.mark.parametrize("order", [0, 1])
def test_sink_strengths(sna, delta, order):
    rep = _case(sna, "sink", 1, 2, 2, 512, 128, True, delta, 1.0, order, 22)
    if delta == 30.0 and order == 0:
        assert rep["underflow_gpu"] > 0.99


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("order", [0, 1])
@pytest.mark.parametrize("S", [1.0, 256.0, 0.0])
def test_random_bias(sna, d, causal, order, S):
    """A bias on about half of all keys: every block takes the general path, and
    the counters skip exactly the biased keys."""
    B, Hq, Hkv, N, seed = 1, 3, 3, 384, 31
    print(f"\n[case] random bias: d={d} causal={causal} order={order} S={S}", flush=True)
    qb, kb, vb = synthetic.qkv_bf16(B, Hq, Hkv, N, d, seed)
    bias = synthetic.random_bias(N, seed)
    out, st = _run(sna, qb, kb, vb, bias, causal, S, order)
    rep = _parity.compare(out, st, qb, kb, vb, bias, causal, S, order)
    print(f"[case] random bias: {rep}", flush=True)


@pytest.mark.parametrize("N", [64, 192])
@pytest.mark.parametrize("order", [0, 1])
def test_partial_workgroups(sna, N, order):
    # 128-row workgroups: N = 64 leaves two waves of the only workgroup without rows,
    # N = 192 the last workgroup half empty; GQA groups of 2
    _case(sna, f"partial N={N}", 3, 6, 3, N, 128, True, 7.0, 256.0, order, 32)


@pytest.mark.parametrize("N", [37, 100, 321])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("order", [0, 1])
def test_ragged_sequence(sna, N, d, causal, order):
    # N not a multiple of 64: the last key block is partial (keys past N masked), the
    # last 64-row counter block short, and rows past N neither stored nor counted
    _case(sna, f"ragged N={N}", 2, 4, 2, N, d, causal, 7.0, 256.0, order, 34)


@pytest.mark.parametrize("S", [1.0, 448.0, 512.0, 3.0, 0.0])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_sequence_scales(sna, S, causal):
    _case(sna, "ragged scales", 1, 2, 1, 200, 128, causal, 7.0, S, 0, 35)


@pytest.mark.parametrize("S", [256.0, 0.0])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_sequence_random_bias(sna, causal, S):
    B, Hq, Hkv, N, d, seed = 1, 3, 3, 150, 128, 36
    print(f"\n[case] ragged random bias: N={N} causal={causal} S={S}", flush=True)
    qb, kb, vb = synthetic.qkv_bf16(B, Hq, Hkv, N, d, seed)
    bias = synthetic.random_bias(N, seed)
    out, st = _run(sna, qb, kb, vb, bias, causal, S, 1)
    rep = _parity.compare(out, st, qb, kb, vb, bias, causal, S, 1)
    print(f"[case] ragged random bias: {rep}", flush=True)


@pytest.mark.parametrize("causal", [False, True])
def test_single_row(sna, causal):
    # N = 1: one query, one key; the output is E4M3(V[0]) exactly
    rep = _case(sna, "one row", 1, 2, 1, 1, 64, causal, None, 256.0, 1, 37)
    assert rep["max_dev"] == 0.0


def _random_configs(n, seed):
    """n seeded mixed configurations: shapes (any N up to 700, grouped kv heads, d 64 / 128),
    mask, order, every conversion mode of S, and no / sink / random bias."""
    rng = np.random.default_rng(seed)
    heads = [(1, 1), (4, 2), (8, 1), (3, 3)]
    scales = [1.0, 2.0, 3.0, 16.0, 256.0, 300.0, 448.0, 512.0, 1000.0, 0.0]
    out = []
    for i in range(n):
        Hq, Hkv = heads[rng.integers(len(heads))]
        out.append(dict(B=int(rng.integers(1, 3)), Hq=Hq, Hkv=Hkv, N=int(rng.integers(1, 701)),
                        d=int(rng.choice([64, 128])), causal=bool(rng.integers(2)), order=int(rng.integers(2)),
                        S=float(rng.choice(scales)), bias=str(rng.choice(["none", "sink", "random"])),
                        delta=float(rng.uniform(0.0, 12.0)), seed=1000 + i))
    return out


@pytest.mark.parametrize("cfg", _random_configs(40, 2024), ids=lambda c: f"N{c['N']}-d{c['d']}-S{c['S']:g}")
def test_random_configurations(sna, cfg):
    c = cfg
    print(f"\n[case] random configuration: {c}", flush=True)
    qb, kb, vb = synthetic.qkv_bf16(c["B"], c["Hq"], c["Hkv"], c["N"], c["d"], c["seed"])
    bias = {"none": None, "sink": synthetic.sink_bias(c["N"], c["delta"]),
            "random": synthetic.random_bias(c["N"], c["seed"])}[c["bias"]]
    out, st = _run(sna, qb, kb, vb, bias, c["causal"], c["S"], c["order"])
    rep = _parity.compare(out, st, qb, kb, vb, bias, c["causal"], c["S"], c["order"])
    print(f"[case] random configuration: {rep}", flush=True)


def test_many_small_heads(sna):
    # a wide grid of short rows: 8 x 16 heads of 128 rows, groups of 4 query heads
    _case(sna, "many heads", 8, 16, 4, 128, 128, False, 7.0, 256.0, 1, 33)


def test_zero_queries_exact_mean(sna):
    """Q = 0: every p = 1, so out = mean of E4M3(V) over the visible keys."""
    print("\n[case] zero queries", flush=True)
    _, kb, vb = synthetic.qkv_bf16(1, 1, 1, 256, 128, 23)
    qb = np.zeros_like(kb)
    out, _ = _run(sna, qb, kb, vb, None, True, 256.0, 1, stats=False)
    vh = torch.from_numpy(vb.view(np.int16)).view(torch.bfloat16).float().to(torch.float8_e4m3fn)
    vh = vh.double().numpy()[0, 0]
    expect = np.cumsum(vh, axis=0) / np.arange(1, 257)[:, None]
    assert np.max(np.abs(out[0, 0] - expect)) < 1e-5


def test_single_block_orders_identical(sna):
    print("\n[case] one key block, both orders", flush=True)
    qb, kb, vb = synthetic.qkv_bf16(2, 2, 2, 64, 128, 24)
    bias = synthetic.sink_bias(64, 7.0)
    a, sa = _run(sna, qb, kb, vb, bias, True, 256.0, 0)
    b, sb = _run(sna, qb, kb, vb, bias, True, 256.0, 1)
    assert np.array_equal(a, b) and np.array_equal(sa, sb)


def test_deterministic_and_stats_do_not_change_output(sna):
    print("\n[case] determinism", flush=True)
    qb, kb, vb = synthetic.qkv_bf16(1, 4, 4, 1024, 128, 25)
    bias = synthetic.sink_bias(1024, 7.0)
    a, sa = _run(sna, qb, kb, vb, bias, True, 256.0, 1)
    b, sb = _run(sna, qb, kb, vb, bias, True, 256.0, 1)
    c, _ = _run(sna, qb, kb, vb, bias, True, 256.0, 1, stats=False)
    assert np.array_equal(a, b) and np.array_equal(sa, sb) and np.array_equal(a, c)


def test_errors_are_reported(sna):
    q = torch.zeros(1, 1, 64, 96, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sna.PcastError) as ei:
        sna.forward(q, q, q, None, S=256.0)
    assert ei.value.code == sna.PCAST_ENOTSUP
    # a caller's out must be a contiguous fp32 [B, Hq, N, d] tensor on the same device
    q = torch.zeros(1, 2, 128, 64, dtype=torch.bfloat16, device="cuda")
    for bad in (torch.empty(1, 2, 128, 64, dtype=torch.bfloat16, device="cuda"),
                torch.empty(1, 2, 64, 64, dtype=torch.float32, device="cuda"),
                torch.empty(1, 2, 64, 128, dtype=torch.float32, device="cuda").transpose(2, 3),
                torch.empty(1, 2, 128, 64, dtype=torch.float32)):
        with pytest.raises(ValueError):
            sna.forward(q, q, q, None, S=256.0, out=bad)


def test_collapse_warning(sna):
    print("\n[case] collapse warning", flush=True)
    q = torch.zeros(1, 1, 128, 64, dtype=torch.bfloat16, device="cuda")
    bias = torch.from_numpy(synthetic.sink_bias(128, 7.0)).cuda()
    with pytest.warns(RuntimeWarning, match="collapse"):
        sna.forward(q, q, q, bias, S=1.0, order="forward", check_collapse=True)
    import warnings
    with warnings.catch_warnings():
        warnings.simplefilter("error")
        sna.forward(q, q, q, bias, S=256.0, order="forward", check_collapse=True)
        sna.forward(q, q, q, bias, S=1.0, order="reverse", check_collapse=True)
    torch.cuda.synchronize()


W = synthetic.WORKLOADS
_INPUTS = {}


def _workload_inputs(name):
    """Q, K, V bits of a workload (generated once per module) and their GPU copies."""
    if name not in _INPUTS:
        _INPUTS.clear()                      # keep one full-size workload in memory at a time
        w = W[name]
        qb, kb, vb = synthetic.qkv_bf16(w.B, w.Hq, w.Hkv, w.N, w.d, w.seed)
        _INPUTS[name] = (qb, kb, vb, tuple(_parity.to_gpu_bf16(x) for x in (qb, kb, vb)))
    return _INPUTS[name]


def _workload_case(sna, name, delta, S, order, blocks):
    w = W[name]
    print(f"\n[case] {name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} d={w.d} causal={w.causal} "
          f"delta={delta} S={S} order={order} seed={w.seed} blocks={len(blocks)}", flush=True)
    qb, kb, vb, (q, k, v) = _workload_inputs(name)
    bias = synthetic.sink_bias(w.N, delta)
    out, st = sna.forward(q, k, v, torch.from_numpy(bias).cuda(), causal=w.causal, S=S, order=order,
                          stats=True)
    torch.cuda.synchronize()
    out_np = out.cpu().numpy()
    st_np = st.cpu().numpy()
    del out, st
    rep = _parity.compare(out_np, st_np, qb, kb, vb, bias, w.causal, S, order, blocks)
    print(f"[case] {name}: {rep}", flush=True)
    return rep


def _sweep_blocks(i):
    """Four 64-row blocks for Sweep cell i: the last block of one head (every key) and three
    more that move with i across heads and positions."""
    return sorted({(0, i % 8, 63), (0, (i + 3) % 8, (5 * i + 11) % 63),
                   (0, (i + 5) % 8, (7 * i + 29) % 63), (0, (i + 6) % 8, (3 * i) % 63)})


@pytest.mark.parametrize("i", range(len(W["sweep"].cases)),
                         ids=[f"d{c[0]:g}-S{c[1]:g}-{'rev' if c[2] else 'fwd'}" for c in W["sweep"].cases])
def test_sweep_cells(sna, i):
    """Every cell of the Sweep (delta 0..10, S = 2^0..2^9 and 448, both orders) on the same
    Q, K, V, four sampled 64-row blocks each."""
    delta, S, order = W["sweep"].cases[i]
    _workload_case(sna, "sweep", delta, S, order, _sweep_blocks(i))


@pytest.mark.parametrize("delta,S,order", W["throughput"].cases)
def test_throughput_full_size(sna, delta, S, order):
    w = W["throughput"]
    _workload_case(sna, "throughput", delta, S, order, _parity.stride_blocks(w.B, w.Hq, w.N, 16))


@pytest.mark.parametrize("delta,S,order", W["gqa"].cases)
def test_gqa_full_size(sna, delta, S, order):
    w = W["gqa"]
    _workload_case(sna, "gqa", delta, S, order, _parity.stride_blocks(w.B, w.Hq, w.N, 64))


@pytest.mark.parametrize("delta,S,order", W["long"].cases)
def test_long_full_size(sna, delta, S, order):
    w = W["long"]
    _workload_case(sna, "long", delta, S, order, _parity.stride_blocks(w.B, w.Hq, w.N, 128))


@pytest.mark.parametrize("qk_fp8", [False, True])
def test_nan_in_one_query_row_stays_in_that_row(sna, qk_fp8):
    """Non-finite inputs give undefined output only where they are seen: a NaN in one row
    of Q leaves every other row of out, and the counters of every other 64-row block,
    bit-identical to the run without it."""
    print(f"\n[case] NaN in one query row, FP8 logits={qk_fp8}", flush=True)
    B, Hq, Hkv, N, d = 1, 2, 1, 256, 128
    qb, kb, vb = synthetic.qkv_bf16(B, Hq, Hkv, N, d, 26)
    bias = torch.from_numpy(synthetic.sink_bias(N, 7.0)).cuda()
    q, k, v = (_parity.to_gpu_bf16(x) for x in (qb, kb, vb))
    qn = q.clone()
    qn[0, 1, 77, 5] = float("nan")
    a, sa = sna.forward(q, k, v, bias, causal=True, S=256.0, order="reverse", stats=True, qk_fp8=qk_fp8)
    b, sb = sna.forward(qn, k, v, bias, causal=True, S=256.0, order="reverse", stats=True, qk_fp8=qk_fp8)
    torch.cuda.synchronize()
    a, b, sa, sb = (x.cpu().numpy() for x in (a, b, sa, sb))
    keep = np.ones((B, Hq, N), dtype=bool)
    keep[0, 1, 77] = False
    assert np.array_equal(a[keep], b[keep])
    keep_st = np.ones(sa.shape[:3], dtype=bool)
    keep_st[0, 1, 77 // 64] = False
    assert np.array_equal(sa[keep_st], sb[keep_st])

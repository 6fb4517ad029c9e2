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
    q = torch.zeros(1, 1, 96, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sna.PcastError) as ei:
        sna.forward(q, q, q, None, S=256.0)
    assert ei.value.code == sna.PCAST_ENOTSUP


SWEEP_CELLS = [(dl, S, o) for dl in (0.0, 5.0, 7.0, 10.0) for S in (1.0, 16.0, 256.0, 448.0, 512.0)
               for o in (0, 1)]


@pytest.mark.parametrize("delta,S,order", SWEEP_CELLS)
def test_sweep_cells(sna, delta, S, order):
    _case(sna, "sweep", 1, 8, 8, 4096, 128, True, delta, S, order, 2, blocks=12)


W = synthetic.WORKLOADS


@pytest.mark.parametrize("delta,S,order", W["throughput"].cases)
def test_throughput_full_size(sna, delta, S, order):
    w = W["throughput"]
    _case(sna, "throughput", w.B, w.Hq, w.Hkv, w.N, w.d, w.causal, delta, S, order, w.seed, blocks=8)


@pytest.mark.parametrize("delta,S,order", W["gqa"].cases)
def test_gqa_full_size(sna, delta, S, order):
    w = W["gqa"]
    _case(sna, "gqa", w.B, w.Hq, w.Hkv, w.N, w.d, w.causal, delta, S, order, w.seed, blocks=6)


@pytest.mark.parametrize("delta,S,order", [(7.0, 256.0, 1), (9.0, 256.0, 0)])
def test_long_full_size(sna, delta, S, order):
    w = W["long"]
    _case(sna, "long", w.B, w.Hq, w.Hkv, w.N, w.d, w.causal, delta, S, order, w.seed, blocks=4)

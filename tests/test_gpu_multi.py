"""The multi-configuration forward (attn_fwd_pcast_multi) against one call per
configuration: the same kernels on the same Q, K, V, so every configuration's output
and counters must be bit-identical to attn_fwd_pcast_prepared's.  The single calls are
themselves checked against the oracle in test_gpu_parity.py."""
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


# every conversion mode (powers of two, 448 and 3 multiply, 512 clamps, 600 multiplies and
# clamps), both orders, with and without a sink, one configuration without any bias
CONFIGS = [(dl, S, o) for dl in (None, 0.0, 7.0) for S in (1.0, 2.0, 256.0, 448.0, 512.0, 3.0, 600.0)
           for o in (0, 1)]


def _check(sna, B, Hq, Hkv, N, d, causal, configs, seed, stats=True):
    print(f"\n[case] multi: B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} causal={causal} cells={len(configs)} "
          f"stats={stats} seed={seed}", flush=True)
    qb, kb, vb = synthetic.qkv_bf16(B, Hq, Hkv, N, d, seed)
    q, k, v = (_parity.to_gpu_bf16(x) for x in (qb, kb, vb))
    biases = [None if dl is None else torch.from_numpy(synthetic.sink_bias(N, dl)).cuda() for dl, _, _ in configs]
    outs, sts = sna.forward_multi(q, k, v, [(bi, S, o) for bi, (_, S, o) in zip(biases, configs)],
                                  causal=causal, stats=stats)
    torch.cuda.synchronize()
    for i, (bi, (dl, S, o)) in enumerate(zip(biases, configs)):
        ref, rst = sna.forward(q, k, v, bi, causal=causal, S=S, order=o, stats=stats)
        torch.cuda.synchronize()
        assert torch.equal(outs[i], ref), f"configuration {i} ({dl}, {S}, {o}): out differs"
        if stats:
            assert torch.equal(sts[i], rst), f"configuration {i} ({dl}, {S}, {o}): counters differ"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_multi_equals_single_calls(sna, d, causal):
    _check(sna, 2, 4, 2, 320, d, causal, CONFIGS, 61)


def test_multi_without_counters(sna):
    _check(sna, 1, 2, 1, 256, 128, True, CONFIGS[:8], 62, stats=False)


def test_multi_more_cells_than_one_launch(sna):
    # 130 configurations of one conversion mode: two launches of that mode (at most 112 each)
    configs = [(float(i % 11), 256.0, i % 2) for i in range(130)]
    _check(sna, 1, 2, 2, 192, 128, True, configs, 63)


def test_multi_sweep_cells(sna):
    """A slice of the Sweep workload (B1 H8 N4096 d128 causal) in one call."""
    w = synthetic.WORKLOADS["sweep"]
    configs = [c for i, c in enumerate(w.cases) if i % 12 == 0]
    _check(sna, w.B, w.Hq, w.Hkv, w.N, w.d, w.causal, configs, w.seed)


@pytest.mark.parametrize("causal", [False, True])
def test_multi_ragged_sequence(sna, causal):
    # N = 200: a partial last key block in every cell
    _check(sna, 1, 2, 1, 200, 128, causal, CONFIGS[::3], 64)

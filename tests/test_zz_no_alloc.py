"""attn_fwd_pcast_noalloc (the forward for callers that cannot allocate) against
attn_fwd_pcast, through the C ABI: the same kernels on the same inputs, so out and
the counters must be bit-identical.  Two calls in a row on one stream, the second
with a smaller input (the scratch keeps the first call's bytes, which the second
must not read), then a third at the first size again; an input above the scratch
limit is rejected before anything is enqueued."""
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


def _run(sna, fn, case, seed):
    B, Hq, Hkv, N, d, causal, S, order = case
    qb, kb, vb = synthetic.qkv_bf16(B, Hq, Hkv, N, d, seed)
    q, k, v = (_parity.to_gpu_bf16(x) for x in (qb, kb, vb))
    bias = torch.from_numpy(synthetic.sink_bias(N, 7.0)).cuda()
    out = torch.full((B, Hq, N, d), float("nan"), dtype=torch.float32, device="cuda")
    st = torch.full((sna.stats_words(B, Hq, N),), -1, dtype=torch.int64, device="cuda")
    rc = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), bias.data_ptr(), B, Hq, Hkv, N, d, causal, S, order,
            out.data_ptr(), st.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == 0, sna.strerror(rc)
    torch.cuda.synchronize()
    return out.cpu().numpy(), st.cpu().numpy()


CASES = [
    (2, 8, 2, 2048, 128, 1, 256.0, 1),   # 2 MiB of scratch
    (1, 2, 1, 192, 64, 0, 1.0, 0),       # smaller, another head size, non-causal, forward
    (1, 4, 4, 256, 128, 1, 0.0, 0),      # the bf16 path (a bf16 V copy)
    (1, 2, 1, 200, 128, 0, 256.0, 1),    # a partial last key block (zero-padded V copy)
    (2, 8, 2, 2048, 128, 1, 448.0, 0),   # the first size again
]


@pytest.mark.parametrize("i", range(len(CASES)))
def test_noalloc_equals_allocating_entry(sna, i):
    case = CASES[i]
    print(f"\n[case] noalloc call {i}: B,Hq,Hkv,N,d,causal,S,order = {case}", flush=True)
    a, sa = _run(sna, sna.attn_fwd_pcast, case, 40 + i)
    b, sb = _run(sna, sna.attn_fwd_pcast_noalloc, case, 40 + i)
    assert not np.isnan(b).any()
    assert np.array_equal(a, b) and np.array_equal(sa, sb)


def test_noalloc_twice_in_a_row_smaller_second(sna):
    """Two calls back to back on one stream, no synchronisation between them."""
    print("\n[case] noalloc: two calls back to back, the second smaller", flush=True)
    big, small = CASES[0], CASES[1]
    ref_big = _run(sna, sna.attn_fwd_pcast, big, 50)
    ref_small = _run(sna, sna.attn_fwd_pcast, small, 51)
    outs = []
    for case, seed in ((big, 50), (small, 51)):
        B, Hq, Hkv, N, d, causal, S, order = case
        qb, kb, vb = synthetic.qkv_bf16(B, Hq, Hkv, N, d, seed)
        q, k, v = (_parity.to_gpu_bf16(x) for x in (qb, kb, vb))
        bias = torch.from_numpy(synthetic.sink_bias(N, 7.0)).cuda()
        out = torch.empty((B, Hq, N, d), dtype=torch.float32, device="cuda")
        st = torch.empty((sna.stats_words(B, Hq, N),), dtype=torch.int64, device="cuda")
        rc = sna.attn_fwd_pcast_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), bias.data_ptr(), B, Hq, Hkv, N,
                                        d, causal, S, order, out.data_ptr(), st.data_ptr(),
                                        torch.cuda.current_stream().cuda_stream)
        assert rc == 0, sna.strerror(rc)
        outs.append((out, st, (q, k, v, bias)))
    torch.cuda.synchronize()
    for (out, st, _), (ra, rs) in zip(outs, (ref_big, ref_small)):
        assert np.array_equal(out.cpu().numpy(), ra) and np.array_equal(st.cpu().numpy(), rs)


def test_noalloc_rejects_inputs_above_the_scratch(sna):
    # B * Hkv * N * d = 2^27 bytes of E4M3 V: twice the scratch.  Checked on the host.
    FAKE = 0x10000
    rc = sna.attn_fwd_pcast_noalloc(FAKE, FAKE, FAKE, 0, 1, 8, 8, 131072, 128, 1, 256.0, 1, FAKE, 0, 0)
    assert rc == sna.PCAST_ENOTSUP
    assert "scratch" in sna.strerror(rc)
    # the largest input that fits: exactly the limit
    assert sna.workspace_bytes(1, 4, 131072, 128, 256.0) == sna.NOALLOC_SCRATCH_BYTES

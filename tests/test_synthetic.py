"""The seeded input generator: deterministic, addressable by slice, N(0,1), bf16 RNE."""
import numpy as np
import torch
from scipy import stats

import synthetic


def test_deterministic_and_sliceable():
    a = synthetic.gaussian_bf16(3, 1, (4, 1000))
    b = synthetic.gaussian_bf16(3, 1, (4, 1000))
    assert np.array_equal(a, b)
    part = synthetic.gaussian_bf16(3, 1, (500,), first=1700)
    assert np.array_equal(a.reshape(-1)[1700:2200], part)
    assert not np.array_equal(a, synthetic.gaussian_bf16(3, 2, (4, 1000)))
    assert not np.array_equal(a, synthetic.gaussian_bf16(4, 1, (4, 1000)))


def test_standard_normal():
    x = synthetic.bf16_bits_to_f32(synthetic.gaussian_bf16(1, 0, (400000,))).astype(np.float64)
    assert abs(x.mean()) < 0.01 and abs(x.var() - 1) < 0.01
    assert stats.kstest(x, "norm").statistic < 0.01   # bf16 rounding shifts the CDF only slightly


def test_values_are_bf16_rounded():
    bits = synthetic.gaussian_bf16(5, 0, (10000,))
    f = synthetic.bf16_bits_to_f32(bits)
    assert np.array_equal(torch.from_numpy(f).to(torch.bfloat16).float().numpy(), f)


def test_sink_bias():
    b = synthetic.sink_bias(128, 7.0)
    assert b.dtype == np.float32 and np.all(b[:4] == 7.0) and np.all(b[4:] == 0)


def test_workload_sizes():
    w = synthetic.WORKLOADS
    assert w["throughput"].flops == 2 * 4 * 32 * 8192 ** 2 * 128
    assert w["tiny"].flops == 4 * 1024 ** 2 * 64
    assert len(w["sweep"].cases) == 11 * 11 * 2


def test_bench_refuses_several_gpus():
    """bench.py measures one GPU: --gpus 2 ends with a message and exit code 2, before any device use."""
    import subprocess
    import sys
    from pathlib import Path
    root = Path(__file__).resolve().parents[1]
    r = subprocess.run([sys.executable, str(root / "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr

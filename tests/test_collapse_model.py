"""The library's collapse-model functions (host code, no GPU) against the oracle's
closed forms (oracle.theory, which is pinned by Monte Carlo of the model)."""
import math

import numpy as np
import pytest

import softmax_numerics_amd as sna
from oracle import theory


@pytest.fixture(scope="module")
def lib():
    import os
    if not os.path.exists(sna.LIB_PATH):
        from softmax_numerics_amd import build
        build.build()
    return sna.load_library()


@pytest.mark.parametrize("k", [1, 2, 3, 4, 8, 16])
def test_sink_max_mean(lib, k):
    assert abs(sna.sink_max_mean(k) - theory.delta_k(k)) < 1e-9
    if k == 1:
        assert abs(sna.sink_max_mean(1)) < 1e-12


@pytest.mark.parametrize("S", [1.0, 16.0, 256.0, 448.0, 512.0])
def test_delta_critical(lib, S):
    want = theory.delta_c(S, 4, threshold=theory.LN2_TEN)
    assert abs(sna.delta_critical(S) - want) < 1e-9
    # the summary's printed thresholds (6.93 + ln S - delta_4), to its rounding
    assert abs(sna.delta_critical(S) - theory.delta_c(S)) < 0.002


@pytest.mark.parametrize("delta", [0.0, 3.0, 5.0, 7.0, 9.0, 12.0])
@pytest.mark.parametrize("S", [1.0, 256.0, 448.0])
def test_underflow_and_lost_mass_models(lib, delta, S):
    f = sna.underflow_model(delta, S)
    assert abs(f - theory.f_exact(delta, S)) < 1e-9 * max(1.0, f) + 1e-15
    g = sna.lost_mass_model(delta, S)
    assert abs(g - theory.f_exact(delta - 1.0, S)) < 1e-9 * max(1.0, g) + 1e-15
    assert g <= f                         # the lost mass sits in the smallest probabilities


def test_known_values(lib):
    assert abs(sna.sink_max_mean(4) - 1.029375373) < 1e-9
    assert abs(sna.delta_critical(1.0) - (10 * math.log(2) - 1.029375373)) < 1e-8
    assert abs(sna.underflow_model(7.0, 1.0) - 0.8156) < 1e-4


def test_bad_arguments_give_nan(lib):
    for v in (sna.delta_critical(0.0), sna.delta_critical(-1.0), sna.delta_critical(float("inf")),
              sna.underflow_model(float("nan"), 1.0), sna.lost_mass_model(7.0, 1.0, 0),
              sna.sink_max_mean(0), sna.sink_max_mean(2000)):
        assert np.isnan(v)


def test_collapse_check(lib):
    """The run-time warning: forward order at S = 1 with the configs' sink (delta 7 on
    keys 0..3) is past Delta_c(1) = 5.90; S = 256 (Delta_c = 11.45) and reverse order
    are not; delta 5 at S = 1 is below the threshold; no bias, no sink."""
    N = 1024
    bias = np.zeros(N, dtype=np.float32)
    bias[:4] = 7.0
    r = sna.collapse_check(bias, 1.0, "forward")
    assert r["collapse"] and r["k"] == 4 and r["delta"] == 7.0
    assert abs(r["delta_c"] - sna.delta_critical(1.0)) < 1e-12
    assert abs(r["underflow"] - sna.underflow_model(7.0, 1.0)) < 1e-12
    assert not sna.collapse_check(bias, 256.0, "forward")["collapse"]
    assert not sna.collapse_check(bias, 1.0, "reverse")["collapse"]
    bias[:4] = 5.0
    assert not sna.collapse_check(bias, 1.0, "forward")["collapse"]
    bias[:4] = 13.0
    assert sna.collapse_check(bias, 448.0, "forward")["collapse"]      # Delta_c(448) = 12.01
    r = sna.collapse_check(None, 1.0, "forward")
    assert not r["collapse"] and r["k"] == 0 and np.isnan(r["delta_c"])
    bias[7] = float("nan")
    with pytest.raises(sna.PcastError):
        sna.collapse_check(bias, 1.0, "forward")

"""Pins for the closed forms of the collapse analysis and the emulator's counters.

* delta_k by quadrature against a direct Monte Carlo of max-of-4 normals and
  against the summary's "about 1.0";
* the underflow fraction the block pipeline produces on logits drawn from the
  model, against the exact model integral F*(Delta, S) (within 4 standard
  errors) and against the summary's plug-in formula (within its own
  approximation error);
* the collapse threshold Delta_c and the reverse-order bound as printed.
"""
import math

import numpy as np
import pytest
from scipy import stats

from oracle import theory


def test_delta_k(golden):
    dk = theory.delta_k(4)
    rng = np.random.default_rng(0)
    mc = rng.standard_normal((2_000_000, 4)).max(axis=1)
    assert abs(dk - mc.mean()) < 4 * mc.std() / math.sqrt(mc.size)
    assert abs(dk - golden["delta_k_approx_k4"]["value"]) < 0.05
    assert theory.delta_k(1) == pytest.approx(0.0, abs=1e-10)
    assert theory.delta_k(2) == pytest.approx(1 / math.sqrt(math.pi), rel=1e-9)   # textbook value


def test_plugin_formula_constants(golden):
    thr = golden["threshold_log_constant"]["value"]
    dk = theory.delta_k(4)
    for delta, S in ((5, 1), (7, 1), (9, 256), (10, 448)):
        expect = stats.norm.cdf(delta + dk - thr - math.log(S))
        assert theory.f_plugin(delta, S) == pytest.approx(expect, rel=1e-12)


@pytest.mark.parametrize("delta,S", [(5, 1), (6, 1), (7, 1), (8, 1), (9, 256), (10, 256), (10, 448),
                                     (8, 4), (6, 2)])
def test_emulator_underflow_matches_model(delta, S):
    fr = theory.monte_carlo_underflow(delta, S, n_keys=1024, n_rows=3000, seed=delta * 1000 + int(S))
    mean, se = fr.mean(), fr.std(ddof=1) / math.sqrt(fr.size)
    fx = theory.f_exact(delta, S)
    assert abs(mean - fx) <= 4 * se + 2e-4
    # the plug-in form approximates F* (Jensen gap): close where F is not tiny
    if fx > 0.01:
        assert abs(theory.f_plugin(delta, S) - fx) < 0.06


def test_collapse_onset(golden):
    lo, hi = golden["collapse_onset_delta"]["range"]
    # plug-in threshold for S = 1, and the exact model crossing 1/2
    dc = theory.delta_c(1.0)
    assert dc == pytest.approx(golden["threshold_log_constant"]["value"] - theory.delta_k(4))
    assert lo - 0.5 < dc < hi
    assert theory.f_exact(lo - 1, 1.0) < 0.5 < theory.f_exact(lo, 1.0) < theory.f_exact(hi, 1.0)
    # larger S moves the threshold up by ln S
    assert theory.delta_c(256.0) - dc == pytest.approx(math.log(256.0))


def test_reverse_order_bound(golden):
    """Reverse order: the running max before the sink block is the non-sink max,
    about sqrt(2 ln N); a non-sink underflows only below that minus 10 ln 2 + ln S."""
    bound = golden["reverse_s256_underflow_bound"]["value"]
    n_max = golden["reverse_s256_underflow_bound"]["n_max"]
    for n in (4096, 131072, n_max):
        p = stats.norm.cdf(math.sqrt(2 * math.log(n)) - theory.LN2_TEN - math.log(256.0))
        assert p < bound
    # whereas forward order at the same S collapses once Delta exceeds ~11.4
    assert theory.f_exact(13.0, 256.0) > 0.5


def test_reverse_order_emulator_has_no_late_underflow():
    """Emulator on model logits, reverse, S = 256: no non-sink outside block 0 rounds to 0."""
    rng = np.random.default_rng(1)
    s = rng.standard_normal((500, 4096))
    s[:, :4] += 9.0
    from oracle.reference import emulate_vectorized
    nonsink = np.ones(4096, dtype=bool)
    nonsink[:4] = False
    nonsink_late = nonsink.copy()
    nonsink_late[:64] = False
    _, _, z_late = emulate_vectorized(s, np.zeros((4096, 1)), 256.0, 1, "pages", 64, nonsink_late)
    _, _, z_late_fwd = emulate_vectorized(s, np.zeros((4096, 1)), 256.0, 0, "pages", 64, nonsink_late)
    assert z_late.sum() == 0
    assert z_late_fwd.sum() > 0          # forward at Delta = 9 already loses some

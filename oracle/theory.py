"""Closed forms of the P-cast collapse analysis, and a Monte Carlo of its model.

Test infrastructure: only the tests use this module.

Model (P-cast summary, section "Metodologia e Analisi"): in natural-log logit
units, non-sink logits are i.i.d. N(0,1); k sink keys carry logit z + Delta
with z ~ N(0,1).  Under forward order the running max applied to every
non-sink key is (about) the largest sink logit, Delta + M_k, with M_k the max
of k standard normals.  A non-sink P = exp(z - Delta - M_k) is cast to zero
when S*P <= 2^-10, i.e. when z <= Delta + M_k - 10 ln 2 - ln S.  Hence

    F*(Delta, S)      = E[ Phi(Delta + M_k - 10 ln 2 - ln S) ]       (exact model)
    F_plug(Delta, S)  = Phi(Delta + delta_k - 6.93 - ln S)           (the summary's formula)

with delta_k = E[M_k] (about 1.0 for k = 4), and the collapse threshold where
the plug-in form crosses 1/2:  Delta_c = 6.93 + ln S - delta_k (summary,
section "Contributi Chiave", point 1).
"""
from __future__ import annotations

import math

import numpy as np
from scipy import integrate, stats

LN2_TEN = 10.0 * math.log(2.0)     # the summary's 6.93
PAGES_THRESHOLD = 6.93              # the constant as printed


def max_normal_pdf(x, k: int):
    """Density of the max of k i.i.d. standard normals."""
    return k * stats.norm.pdf(x) * stats.norm.cdf(x) ** (k - 1)


def delta_k(k: int = 4) -> float:
    """E[max of k i.i.d. N(0,1)] by quadrature."""
    val, _ = integrate.quad(lambda x: x * max_normal_pdf(x, k), -np.inf, np.inf,
                            epsabs=1e-13, epsrel=1e-13)
    return val


def f_exact(delta: float, S: float, k: int = 4) -> float:
    """F*(Delta, S) = E[Phi(Delta + M_k - 10 ln 2 - ln S)]."""
    shift = delta - LN2_TEN - math.log(S)
    val, _ = integrate.quad(lambda x: stats.norm.cdf(shift + x) * max_normal_pdf(x, k),
                            -np.inf, np.inf, epsabs=1e-15, epsrel=1e-12, limit=200)
    return val


def f_plugin(delta: float, S: float, k: int = 4, threshold: float = PAGES_THRESHOLD) -> float:
    """The summary's F(Delta, S) = Phi(Delta + delta_k - 6.93 - ln S)."""
    return float(stats.norm.cdf(delta + delta_k(k) - threshold - math.log(S)))


def delta_c(S: float, k: int = 4, threshold: float = PAGES_THRESHOLD) -> float:
    """Collapse threshold Delta_c = 6.93 + ln S - delta_k."""
    return threshold + math.log(S) - delta_k(k)


def monte_carlo_underflow(delta: float, S: float, n_keys: int, n_rows: int, seed: int,
                          k: int = 4, bc: int = 64, order: int = 0):
    """Run the block pipeline (fp64, exact E4M3) on logits drawn from the model.

    Keys 0..k-1 are sinks (N(0,1) + delta); the others are N(0,1).  Returns the
    per-row underflow fractions of the non-sink keys (code == 0 after the
    cast), so the caller can form a mean and a standard error.
    """
    from .reference import emulate_vectorized
    rng = np.random.default_rng(seed)
    s = rng.standard_normal((n_rows, n_keys))
    s[:, :k] += delta
    nonsink = np.ones(n_keys, dtype=bool)
    nonsink[:k] = False
    v = np.zeros((n_keys, 1))
    _, total, zero = emulate_vectorized(s, v, S, order, "pages", bc, nonsink)
    return zero / total

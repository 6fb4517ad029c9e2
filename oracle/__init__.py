"""CPU oracle for FP8 P-cast attention.

TEST INFRASTRUCTURE.  Only ``tests/``, the smoke check in
``__graft_entry__.py`` and the CPU-baseline leg of ``bench.py`` may import
this package.  It is written from the P-cast summaries and the
FlashAttention blog, in fp64, and shares no code with the HIP path
(``softmax_numerics_amd``); neither imports the other.  The product path
never falls back to it.

Contents
* ``e4m3``      software OCP E4M3 (RNE, saturating at 448) and bf16 rounding
* ``reference`` NumPy fp64 exact attention (O1) and the P-cast block pipeline
                (O2), sequential and telescoped forms
* ``core``      the same O1/O2 in C (pcast_oracle.c, OpenMP), for large inputs,
                with per-row parity slack and underflow counters
* ``qk8``       the FP8-logits extension: power-of-two block scales (per query
                row, per 64-key block) and E4M3 rounding of Q and K
* ``rowdiag``   per-row log-sum-exp and lost non-sink mass of the pipeline
* ``decode``    decode rows with the keys in ranges that each run the pipeline,
                merged by the online-softmax rescale
* ``backward``  gradients by recomputation from the log-sum-exp (cast passed
                straight through)
* ``theory``    the closed forms F(Delta, S), delta_k, Delta_c and a Monte Carlo
                of the collapse model

Parity pins: every function here is checked by ``tests/test_oracle_*.py``
against facts fixed by the pages or by mathematics (see the test docstrings).
"""

from . import backward, decode, e4m3, qk8, reference, rowdiag, theory  # noqa: F401

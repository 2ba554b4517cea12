"""CPU oracle for block-scaled FP8 attention with the Delta-Matching row correction.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, FP64 (numpy)
statement of what the HIP library computes.  Only the tests, the smoke check
and the benchmark's CPU-baseline leg may import it; the library and its Python
binding never do, and the two share no code.

Modules
-------
fp8        OCP E4M3FN / E5M2 codec written from the format definitions, the
           power-of-two 1x32 block quantizer, and the ambiguity bound of casts
           whose input the kernel computes in FP32.
attention  forward (O, LSE), the three row-correction modes (stale,
           dO-matched, matched) and the backward (dQ, dK, dV, row-sum probes),
           with the first-order radius that ambiguous in-kernel casts may move
           a correct kernel result by.

Parity pins: every function here is checked by the ``-m "not gpu"`` tests
against a library routine, a closed form, an exact identity from the Delta-
Matching project page, finite differences or brute force.  The one reading the
pages do not fix -- which running maximum the forward's probability cast uses
(the exact row maximum updated every 128 keys) -- is pinned by a brute-force
streaming implementation in the tests, not by the pages ("parity unpinned" by
the source for that reading alone).
"""
from . import fp8, attention  # noqa: F401

"""Plain fp64 CPU oracle for exact attention.

TEST INFRASTRUCTURE ONLY.  This package is the independent checker for the HIP
path: only the test suite, the smoke check and the benchmark's CPU-baseline leg
may import it.  It shares no code with the HIP library or its Python binding and
imports neither; the product path never routes through it.

Modules
-------
naive        the definition of scaled-dot-product attention and its gradient,
             written out in float64 with library matmuls (the oracle proper).
tiled_model  the pages' tiled FlashAttention-2 forward/backward in float64 with
             counters on every value moved between "HBM" and "SRAM" and on
             every tile visited: a test aid that reproduces the pages' traffic
             and tile counts; it is checked against `naive`, never the reverse.
"""
from . import naive, tiled_model  # noqa: F401

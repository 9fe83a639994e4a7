"""CPU oracle for paged attention -- TEST INFRASTRUCTURE ONLY.

Plain, slow, fp64 NumPy code that states what the paged attention path computes.
Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
it; the library path never does.  It shares no code with the HIP kernels or
their host layer, and imports nothing from the product package.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(brute force, a library attention routine, closed forms, invariances and the
pages' own KV-size arithmetic).  None is "parity unpinned".
"""

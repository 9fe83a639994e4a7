"""CPU oracle for paged attention -- TEST INFRASTRUCTURE ONLY.

Plain, slow, fp64 NumPy code that states what the paged attention path computes.
Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
it; the library path never does.  It shares no code with the HIP kernels or
their host layer, and imports nothing from the product package.

Modules: ``paged_attention`` (gather through the block table, then textbook
softmax attention) and ``kv_cache`` (appending new tokens' K/V into their
slots, block copies, and a reference model of the block pool with shared
blocks and copy-on-write).

Parity status: every function here is pinned.  ``tests/test_oracle_pins.py``
pins the attention oracle (brute force, a library attention routine, closed
forms, invariances and the pages' own KV-size arithmetic);
``tests/test_kv_cache_oracle.py`` pins the append and block copies against the
pinned gather and the pool model against the pages' paging and sharing
statements.  None is "parity unpinned".
"""

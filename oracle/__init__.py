"""CPU oracle for paged decode attention: test infrastructure, not product.

Plain, slow, obviously correct NumPy code in float64 that restates what the
pages define.  Only the test suite, the smoke check and the benchmark's CPU
baseline may import it; the HIP library never does, and this package imports
nothing from the HIP side.

  attention   gather through the block table, then standard softmax attention;
              the per-partition (m, l, o) partials and their log-sum-exp merge
  cache_ops   the slot-mapping scatter of new K/V, and whole-block copies
  quant       the 8-bit KV codes (FP8 E4M3, int8): encode with per-pool
              scales, decode
  allocator   the block pool: FIFO free list, per-block refcounts, fork,
              append with copy-on-write, free

Every function is pinned by the CPU tests (tests/test_oracle_*.py) to closed
forms, invariants, an independent library attention, brute force on tiny
inputs and the worked examples the pages print (tests/golden/).
"""
from . import allocator, attention, cache_ops, quant  # noqa: F401

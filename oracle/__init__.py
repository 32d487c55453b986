"""CPU oracle for the RadixAttention hot path.  TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the bench's CPU-baseline leg may import
anything from this package.  The product library never calls it and shares
no code with it.

What it holds (each function cites the passage it follows):

* ``radix_tree`` -- a deliberately naive radix tree over a FIFO token-slot
  pool: longest-prefix match that splits a partially matched edge, insert
  with edge split, reference-count locks on the root path, and LRU leaf
  eviction done by a linear scan.
* ``attention`` -- causal scaled-dot-product attention in float64, evaluated
  from freshly regenerated Q/K/V for every position (no pool, no cache).
* ``kv_store`` -- the pool after a scatter of new rows.
* ``fp8`` -- the FP8 (OCP E4M3) pool format: codes, rounding, the stored
  values that attention then reads.
* ``hit_rate`` -- token-weighted cache hit rate and the Theorem 3.1 optimum.
* ``runner`` -- the batch scheduler that drives the naive tree through a
  workload and records every observable decision.

Parity status: every function here is pinned by a CPU test against values
the pages fix, closed forms, or brute force (tests/test_oracle_*.py),
except the scheduler's own policy choices (FIFO free order, LRU tie-break,
evict-on-deficit, admission order), which the pages leave open; for those
the parity is self-pinned (oracle and library must agree, no page decides).
"""

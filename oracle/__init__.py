"""The CPU oracle of one DP rank's sharded Adam step.

TEST INFRASTRUCTURE, not part of the product. Only tests/, the smoke check in
__graft_entry__ and bench.py's cpu_baseline leg may import, call, link or run
anything in this package; the HIP path (zero_distributed_optimizer_amd) never
does, and the two share no code, headers, tables or helpers. The seeded input
generators in workloads.py are the only thing both sides use.

  oracle.layout   buckets, padding, rank ranges, the four-way range map (Python)
  oracle.step     the rank's step composed per piece (Python)
  oracle.numerics ctypes front of oracle/step.c, the element arithmetic (C)

Every function is pinned by tests/test_oracle_*.py against what the pages and
the mathematics fix; no function is "parity unpinned".
"""

"""CPU oracle for the DARTree draft-tree construction round.

Test infrastructure only: the tests, the smoke check and the benchmark's
CPU-baseline leg may use it; the product path must not.
"""

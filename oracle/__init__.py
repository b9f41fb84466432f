"""CPU oracle for the batched routed-MoE FFN (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.
"""

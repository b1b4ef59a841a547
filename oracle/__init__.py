"""CPU oracle for the MoE layer (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
this package.  The HIP path never imports it.
"""

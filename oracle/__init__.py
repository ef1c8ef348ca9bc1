"""CPU oracle for the SSB phase-variance objective (float64, test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may import
this package; the GPU library never does.
"""

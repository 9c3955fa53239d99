"""CPU oracle for block-scaled 4-bit quantization.

Test infrastructure only: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the quantization library never does.
"""

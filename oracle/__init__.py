"""Float64 CPU oracle for the selective-scan path.

Test infrastructure only: the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import it; the product path never does.
"""

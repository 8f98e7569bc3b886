"""CPU oracle for index-selected sparse attention (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg use
this package. The GPU library never imports, links or calls it.
"""

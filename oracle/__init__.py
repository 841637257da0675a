"""fp64 CPU oracle for SepLLM separator-mask attention and SepCache.

Test infrastructure only: the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import it; the GPU library never does.
"""

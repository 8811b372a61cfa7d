"""fp64 CPU oracle for sparse paged decode attention.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg.  It shares no code with the HIP library and does
not import it.
"""

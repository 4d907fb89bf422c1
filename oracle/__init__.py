"""fp64 CPU oracle for the patch-pipelined DiT stage.

TEST INFRASTRUCTURE ONLY: imported by the test-suite, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It shares no code with
the HIP library.
"""
from . import ref, brute  # noqa: F401

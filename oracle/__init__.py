"""CPU oracle for the SPIN decode step -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product path (the HIP library and its Python binding) never
imports, links or calls anything here.
"""
from .spin_oracle import *  # noqa: F401,F403

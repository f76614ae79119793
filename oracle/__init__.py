"""CPU fp64 oracle for Token Radius Attention.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg.  The product path (the HIP library and its
Python binding) never imports, calls or links anything here.
"""
from .tra_oracle import *  # noqa: F401,F403

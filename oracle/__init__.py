"""Plain fp64 CPU oracle for the S4 DPLR convolution-mode forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only the tests, the smoke check and the CPU-baseline leg
of the benchmark use it.  It shares no code with the HIP implementation.

See ``oracle/s4.py`` for the functions and the passages each one follows.
"""
from .s4 import *  # noqa: F401,F403

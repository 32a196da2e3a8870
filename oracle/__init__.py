"""fp64 CPU oracle for MLA absorbed decode -- test infrastructure only.

Only the test-suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The library and its binding never do, and the oracle
imports nothing from them.
"""
from .mla_oracle import *  # noqa: F401,F403
from . import mla_oracle  # noqa: F401

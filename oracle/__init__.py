"""CPU oracle for dual-view blocked SpMSpV — test infrastructure only.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The HIP library never calls it and shares no code with
it.  See ``oracle.c`` for the definitions and their citations.
"""
from .oracle import *  # noqa: F401,F403

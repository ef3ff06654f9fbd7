"""CPU oracle for the FlashLoop lazy-update loop step.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this package.  It shares no code with
the HIP path and must never be used as a fallback for it.
"""
from .flashloop_oracle import *  # noqa: F401,F403

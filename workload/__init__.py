"""Seeded synthetic inputs shared by the fp64 oracle tests and the HIP library's
tests and benchmark.  Holds random draws, the INT4-g128 base quantiser and the
canonical packer only; none of the correction method's arithmetic."""
from .gen import *  # noqa: F401,F403

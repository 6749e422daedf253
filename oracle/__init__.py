"""CPU reference for the SparsePR attention call.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and
the CPU-baseline leg of the benchmark, never by the product path.
"""
from .sparsepr_oracle import *  # noqa: F401,F403
from .sparsepr_oracle import __all__  # noqa: F401
from . import rcp  # noqa: F401,E402  response-coupled partitioning

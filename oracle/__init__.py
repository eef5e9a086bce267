"""Float64 CPU oracle of the HSA + HKV forward.

TEST INFRASTRUCTURE: only tests/, the smoke check and the bench's CPU
baseline may import this package; the product path never does.
"""
from .hsa import *  # noqa: F401,F403
from .hsa import __all__  # noqa: F401

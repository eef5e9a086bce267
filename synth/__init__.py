"""Seeded synthetic workloads shared by the oracle checks, the GPU tests and the bench."""
from .inputs import *  # noqa: F401,F403
from .inputs import __all__  # noqa: F401

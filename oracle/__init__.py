"""Float64 CPU oracle of the head-to-neuron affinity pass.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  See affinity.py.
"""
from .affinity import *  # noqa: F401,F403
from .affinity import __all__  # noqa: F401

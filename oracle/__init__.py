"""Float64 CPU oracle of the head-to-neuron affinity pass.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  See affinity.py
(the affinity scores) and objective.py (the layout objective).
"""
from .affinity import *  # noqa: F401,F403
from .affinity import __all__ as _aff_all
from .objective import *  # noqa: F401,F403
from .objective import __all__ as _obj_all

__all__ = list(_aff_all) + list(_obj_all)

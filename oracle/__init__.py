"""Float64 CPU oracle of the head-to-neuron affinity pass.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  See affinity.py
(the affinity scores), objective.py (the layout objective) and
layout_search.py (the layout search) and loo.py (the exact leave-one-out
score).
"""
from .affinity import *  # noqa: F401,F403
from .affinity import __all__ as _aff_all
from .objective import *  # noqa: F401,F403
from .objective import __all__ as _obj_all
from .layout_search import *  # noqa: F401,F403
from .layout_search import __all__ as _ls_all
from .loo import *  # noqa: F401,F403
from .loo import __all__ as _loo_all

__all__ = list(_aff_all) + list(_obj_all) + list(_ls_all) + list(_loo_all)

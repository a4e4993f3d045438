"""CPU oracle of the dropless-MoE expert layer (fp64 numpy).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check and by
the benchmark's CPU-baseline leg, never by the product path.  See
``oracle/dmoe.py`` for the sources each function follows and the pins that
check it.
"""
from .dmoe import *  # noqa: F401,F403
from .dmoe import __all__  # noqa: F401
from . import router  # noqa: F401  (the router in front of the layer)
from . import token_round as rounding  # noqa: F401  (tile-aware token rounding)
from . import moa  # noqa: F401  (dMoA map / reduce)

"""Float64 CPU oracle of the fixed-budget evict-and-attend decode step.

TEST INFRASTRUCTURE: only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import it. See ``kvevict_oracle``.
"""
from .kvevict_oracle import *  # noqa: F401,F403
from .kvevict_oracle import __all__  # noqa: F401

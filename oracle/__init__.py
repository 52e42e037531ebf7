"""CPU oracle of the SLoPe 2:4 sparse linear layer (test infrastructure only).

Only the test suite, the entry module's smoke check and the benchmark's CPU
baseline may import this package.  It shares no code with the GPU library.
"""
from .slope_ref import *  # noqa: F401,F403
from .slope_ref import __all__  # noqa: F401

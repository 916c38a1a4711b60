"""fp64 CPU oracle (test infrastructure only; see oracle.attention)."""

from .attention import *  # noqa: F401,F403
from .attention import __all__  # noqa: F401

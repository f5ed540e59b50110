"""CPU oracle (test infrastructure only; see fp8bs_oracle's docstring)."""
from .fp8bs_oracle import *  # noqa: F401,F403
from .fp8bs_oracle import __all__  # noqa: F401

"""CPU oracle (test infrastructure only; see fp8_oracle's module docstring)."""
from .fp8_oracle import *  # noqa: F401,F403
from .fp8_oracle import Ring  # noqa: F401

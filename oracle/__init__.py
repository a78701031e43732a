"""CPU fp64 oracle (test infrastructure only; see kvp_oracle's header)."""
from .kvp_oracle import *  # noqa: F401,F403

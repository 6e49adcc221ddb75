"""CPU oracle (test infrastructure only; see absh_oracle's header)."""
from .absh_oracle import *  # noqa: F401,F403

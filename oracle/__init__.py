"""CPU oracle (test infrastructure only; see museattn_oracle's header)."""
from .museattn_oracle import *  # noqa: F401,F403

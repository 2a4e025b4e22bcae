"""CPU oracle (test infrastructure only; see ultragen_oracle's header)."""
from .ultragen_oracle import *  # noqa: F401,F403

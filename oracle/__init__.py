"""CPU oracle (test infrastructure only; see herald_oracle)."""
from .herald_oracle import *  # noqa: F401,F403

"""CPU fp64 oracle (test infrastructure only; see uhla_oracle.py)."""
from .uhla_oracle import *  # noqa: F401,F403

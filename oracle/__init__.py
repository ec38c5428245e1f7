"""Float64 CPU oracle (test infrastructure only; see oracle.py)."""
from .oracle import *  # noqa: F401,F403

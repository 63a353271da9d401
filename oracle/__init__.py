"""Plain float64 CPU oracle (test infrastructure only; see gau_oracle)."""
from .gau_oracle import *  # noqa: F401,F403

"""fp64 CPU oracle (test infrastructure only; see muon_oracle.py)."""
from .muon_oracle import *  # noqa: F401,F403

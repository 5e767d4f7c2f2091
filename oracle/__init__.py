"""fp64 CPU oracle for the Muon update step (test infrastructure only)."""
from .muon_oracle import *  # noqa: F401,F403

"""CPU fp64 oracle of the CSA2 read path: test infrastructure only (see csa2_oracle)."""
from .csa2_oracle import *  # noqa: F401,F403

"""CPU oracle of the CSA hot path (test infrastructure only; see csa_oracle's header)."""
from .csa_oracle import *  # noqa: F401,F403

"""fp64 CPU oracle of the DSA decode path (test infrastructure only; see dsa_oracle)."""
from .dsa_oracle import *  # noqa: F401,F403

"""CPU oracle (test infrastructure only; see vsa_oracle.py's header)."""
from .vsa_oracle import *  # noqa: F401,F403

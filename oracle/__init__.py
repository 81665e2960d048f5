"""CPU oracle (test infrastructure only; see tabit_oracle's header)."""
from .tabit_oracle import *  # noqa: F401,F403

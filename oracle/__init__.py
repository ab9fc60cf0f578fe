"""CPU oracle (test infrastructure only; see omni_oracle's header)."""
from .omni_oracle import *  # noqa: F401,F403

"""CPU oracle (test infrastructure only; see ridgefill_oracle's header)."""
from .ridgefill_oracle import *  # noqa: F401,F403
from .ridgefill_oracle import __all__  # noqa: F401

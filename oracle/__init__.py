"""Float64 CPU oracle (test infrastructure only; see kvq_oracle's header)."""
from .kvq_oracle import *  # noqa: F401,F403
from . import kvq_oracle  # noqa: F401

"""CPU oracle package (test infrastructure only; see cacheblend_oracle)."""
from .cacheblend_oracle import *  # noqa: F401,F403

"""CPU oracle (test infrastructure only; see ``quip_oracle``)."""
from .quip_oracle import *  # noqa: F401,F403
from .quip_oracle import NotPositiveDefinite  # noqa: F401

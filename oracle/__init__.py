"""CPU oracle (test infrastructure only; see mpb_oracle's header)."""
from .mpb_oracle import *  # noqa: F401,F403
from . import mpb_oracle  # noqa: F401

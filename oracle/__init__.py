"""CPU oracle (test infrastructure only; see signrot_oracle)."""

from .signrot_oracle import *  # noqa: F401,F403
from . import signrot_oracle  # noqa: F401

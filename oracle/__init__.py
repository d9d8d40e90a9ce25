"""CPU oracle (test infrastructure only; never imported by the product path)."""

from .csa_oracle import *  # noqa: F401,F403
from .csa_oracle import READINGS  # noqa: F401

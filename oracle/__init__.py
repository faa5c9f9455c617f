"""CPU oracle (test infrastructure only; never imported by the product path)."""

from .tq_oracle import *  # noqa: F401,F403
from .tq_oracle import __all__  # noqa: F401

"""CPU oracle (test infrastructure; never imported by the product path)."""
from .hs_oracle import *  # noqa: F401,F403
from .hs_oracle import __all__  # noqa: F401

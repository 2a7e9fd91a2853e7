"""Float64 CPU oracle (test infrastructure only; never imported by the product path)."""
from .g4_oracle import *  # noqa: F401,F403

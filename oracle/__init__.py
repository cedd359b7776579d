"""CPU oracle for the Flint MoE FFN block (test infrastructure only; see flint_oracle)."""
from .flint_oracle import *  # noqa: F401,F403

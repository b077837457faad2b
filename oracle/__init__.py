"""fp64 CPU oracle for the AWQ hot path (test infrastructure only; see awq_oracle)."""
from .awq_oracle import *  # noqa: F401,F403
from . import awq_oracle  # noqa: F401

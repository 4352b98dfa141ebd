"""fp64 CPU oracle for ZHA decode — test infrastructure only (see zha_oracle)."""
from .zha_oracle import *  # noqa: F401,F403

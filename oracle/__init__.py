"""fp64 CPU oracle (test infrastructure only; never imported by the HIP library)."""
from .mla_oracle import *  # noqa: F401,F403

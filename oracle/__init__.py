"""Float64 CPU oracle for causal SATA (test infrastructure only; see sata_oracle)."""
from .sata_oracle import *  # noqa: F401,F403

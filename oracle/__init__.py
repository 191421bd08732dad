"""CPU oracle of the MSA forward path (test infrastructure only; see msa_oracle)."""
from .msa_oracle import *  # noqa: F401,F403

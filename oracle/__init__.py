"""CPU oracle (test infrastructure only): see dsa_oracle.py."""
from . import dsa_oracle  # noqa: F401

"""CPU oracle (test infrastructure only; see fp4_oracle)."""
from . import fp4_oracle  # noqa: F401

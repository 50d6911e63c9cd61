"""CPU oracle of the CSA / HCA step (test infrastructure only; see csa_oracle)."""
from . import csa_oracle  # noqa: F401

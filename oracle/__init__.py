"""fp64 CPU oracle of AQUA attention: test infrastructure only (never on the product path)."""
from . import aqua_oracle  # noqa: F401

"""CPU oracle (test infrastructure only; never imported by the product path)."""
from . import moe_oracle  # noqa: F401

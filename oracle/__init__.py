"""CPU oracle (test infrastructure only; see moe_oracle's header)."""
from . import moe_oracle  # noqa: F401

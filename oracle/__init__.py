"""CPU oracle (test infrastructure only; see awq_oracle's header)."""
from . import awq_oracle  # noqa: F401

"""CPU oracle (test infrastructure only; see ffn_oracle)."""
from . import ffn_oracle  # noqa: F401

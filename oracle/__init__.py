"""CPU oracle (test infrastructure only; see kvq_oracle's docstring)."""
from . import kvq_oracle  # noqa: F401

"""CPU oracle (test infrastructure only; never on the product path)."""
from . import wkv_oracle  # noqa: F401

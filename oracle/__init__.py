"""CPU oracle package (test infrastructure only; see oracle/oracle.py)."""
from . import oracle  # noqa: F401

"""CPU oracle (test infrastructure only: tests, smoke() and bench.py's
cpu_baseline may use it; the GPU library never does)."""
from . import dsa_oracle  # noqa: F401

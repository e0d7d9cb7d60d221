"""CPU oracle of the ZHA decode hot path (NumPy, float64).  Test infrastructure only:
imported by tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg, never by the
product library or its binding."""
from . import zha_oracle  # noqa: F401

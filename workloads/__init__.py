"""Seeded synthetic workloads (shapes and random inputs) shared by tests and benchmarks.
Holds no arithmetic of the method itself."""
from . import configs, gen  # noqa: F401

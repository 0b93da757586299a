"""Seeded synthetic workload generators shared by the oracle tests and the HIP path."""
from . import gen  # noqa: F401

"""Seeded synthetic workloads (sizes, seeds, random draws) for the Sep-Attention hot path."""
from . import configs, gen  # noqa: F401

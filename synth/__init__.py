"""Seeded synthetic inputs and workload shapes (no method arithmetic)."""
from . import configs, gen  # noqa: F401

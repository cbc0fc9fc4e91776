"""Seeded synthetic inputs and workload definitions (no method arithmetic)."""
from . import configs, gen  # noqa: F401

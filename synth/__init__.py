"""Seeded synthetic inputs (no method arithmetic)."""
from . import gen  # noqa: F401

"""Bounds-checked tile movement for MI355X (gfx950)."""
from . import inputs  # noqa: F401

"""Seeded synthetic input generators (no method arithmetic)."""
from .kv_inputs import *  # noqa: F401,F403

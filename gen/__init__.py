"""Seeded synthetic workloads for the sparse-MLA paged decode (inputs only)."""
from .synth import *  # noqa: F401,F403

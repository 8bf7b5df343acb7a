"""Seeded synthetic SGMV workloads (input generation only)."""
from .synth import *  # noqa: F401,F403
from .synth import Problem, F16, BF16, DTYPES  # noqa: F401

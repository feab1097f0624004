"""Synthetic, seeded inputs with the shapes of the pages' workloads.

Shared by the tests, the bench and the oracle checks; it draws and formats
inputs only and contains no step of the method itself.
"""
from .configs import (ALL, BY_NAME, Workload, TINY, V01_UNIT, V02_RANK, V02_WHOLE,  # noqa: F401
                      AUDIO_LONG, V02_PREFILL, JOINT_RANK, STREAMING)
from . import gen  # noqa: F401

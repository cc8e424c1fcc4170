"""Seeded synthetic inputs shared by the oracle-side tests and the GPU-side tests.

This package holds only input generation: seeded random draws and their
rounding to a storage dtype. It holds none of the optimizer's arithmetic.
"""
from .inputs import *  # noqa: F401,F403

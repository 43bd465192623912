"""Seeded synthetic workloads shared by the oracle side and the GPU side."""
from .inputs import *  # noqa: F401,F403
from .inputs import WORKLOADS, Workload, scaled  # noqa: F401

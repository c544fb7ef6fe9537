"""Seeded synthetic workloads shared by the tests, the bench and the oracle.

Holds shapes, distributions and random draws only: none of the attention
block's arithmetic lives here.
"""

from .configs import WORKLOADS, Workload, Layer, LOCAL_SLIDING, GLOBAL, scaled  # noqa: F401
from . import inputs  # noqa: F401

"""Seeded synthetic inputs for paged decode attention.

This package only draws inputs: sequence lengths, physical block ids, block
tables, queries and the K/V token stream that fills the cache.  It holds none
of the method's arithmetic (no gather, no softmax, no quantisation); both the
CPU oracle and the HIP path consume what it produces.
"""

from .configs import CONFIGS, WorkloadConfig, get_config  # noqa: F401
from .generate import Workload, make_workload  # noqa: F401

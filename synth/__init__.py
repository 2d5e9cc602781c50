"""Seeded synthetic inputs for paged decode and prefill attention.

This package only draws inputs: sequence lengths, physical block ids, block
tables, queries and the K/V token stream that fills the cache.  It holds none
of the method's arithmetic (no gather, no softmax, no quantisation); both the
CPU oracle and the HIP path consume what it produces.
"""

from .configs import (CONFIGS, PREFILL_CONFIGS, WorkloadConfig, get_config,  # noqa: F401
                      get_prefill_config)
from .generate import PrefillRows, Workload, make_prefill_rows, make_workload  # noqa: F401

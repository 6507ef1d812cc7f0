"""Seeded synthetic workloads for paged attention.

This package only *draws* inputs: sequence lengths, K/V/Q values in their
storage dtype, physical block placement, block tables and slot mappings.  It
holds none of the method's arithmetic (no dtype encoding, no attention), so
that the oracle and the HIP path can both consume its output without sharing
any code.  See ``workloads.generate`` for the recipe.
"""

from .generate import (  # noqa: F401
    Workload,
    CONFIGS,
    make,
    poison_pattern,
    DTYPE_BYTES,
)
from .accounting import (  # noqa: F401
    kv_bytes_per_token_model,
    workload_kv_bytes,
    workload_pairs,
    workload_flops,
    step_other_bytes,
    fragmentation,
)

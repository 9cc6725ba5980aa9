"""Seeded synthetic decode-attention workloads.

This module only draws random numbers and lays them out in the cache layouts
the kernels and the oracle both read. It holds none of the attention
arithmetic, so that the HIP path and the CPU oracle can share inputs without
sharing any computation.
"""

from .synth import (  # noqa: F401
    quantize_kv_fp8,
    CONFIG_NAMES,
    Workload,
    make_append,
    make_config,
    make_prefill,
    make_workload,
    poison_value,
)

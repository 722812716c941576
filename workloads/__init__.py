"""Seeded synthetic inputs for paged KV-cache writes and paged attention.

This package draws the inputs that both the HIP path and the CPU oracle consume: sequence lengths,
block tables, slot mappings, pool contents and this step's new K/V and Q. It computes nothing of the
attention itself and imports neither the oracle nor the product package.
"""

from .synth import (  # noqa: F401
    BF16,
    FP32,
    Step,
    Workload,
    bf16_bits_from_f32,
    build_workload,
    config_decode,
    config_mixed,
    config_prefix,
    config_spec,
    config_tiny,
    make_config,
    subset_workload,
    CONFIG_NAMES,
)

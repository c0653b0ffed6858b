"""Seeded synthetic inputs for the NVFP4 paged KV cache.

This package only draws random numbers and lays them out (lengths, block
tables, slot mappings, bf16 K/V/Q, the per-tensor kv scale of the recipe).
It holds none of the cache's arithmetic, so both the HIP path and the CPU
oracle can take their inputs from it.
"""
from .gen import Workload, make_workload, make_config, make_activations, fp8_kv_scales, CONFIG_NAMES  # noqa: F401

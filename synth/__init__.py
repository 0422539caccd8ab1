"""Seeded synthetic KV-cache workloads.

This package only draws random numbers and lays them out; it holds none of the
quantisation or attention arithmetic.  Both the CPU oracle (``oracle/``) and the
HIP path (``kv_cache_bit_fwht_amd``) read their inputs from here, so the two
sides see byte-identical fp16 K/V, queries and causal lengths.
"""
from .workloads import (  # noqa: F401
    WORKLOADS,
    Workload,
    get,
    gen_unit,
    gen_kv,
    gen_queries,
    unit_rng,
)

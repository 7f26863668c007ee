"""Seeded synthetic workloads for paged-KV attention (inputs only).

This package draws random numbers and integer layouts (lengths, page
permutations, block tables, slot mappings).  It holds none of the
attention arithmetic and none of the storage-dtype conversions: values are
float32 draws, integers are int32/int64.  Both the CPU oracle (through the
tests) and the GPU path consume what it returns.
"""
from .gen import CONFIGS, Workload, make_workload, custom_workload  # noqa: F401

"""Seeded synthetic inputs (lengths, block tables, q/K/V values) shared by the
tests, the benchmark and the smoke check.  Holds no attention arithmetic."""
from .allocator import BlockAllocator, PoolExhausted, TableEntry  # noqa: F401
from .configs import (CONFIGS, FP8_NAN, Tables, build_tables, duplicate_shared, empty_pools,  # noqa: F401
                      make_fp8_pools, make_history, make_pools, make_query, nan_bits, normal_16bit,
                      random_e4m3, to_bits, torch_dtype)

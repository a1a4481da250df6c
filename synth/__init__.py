"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

Holds no arithmetic of the method: lengths, page tables, slot mappings, random
Q/K/V and NaN poison only.
"""

from .blocks import BLOCK_SIZE, BlockPool, PoolExhausted, blocks_for, slot_of  # noqa: F401
from .workloads import CONFIGS, DecodeConfig, Workload, make_workload, bits_np, NAN_BITS  # noqa: F401

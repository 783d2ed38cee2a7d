"""Seeded synthetic inputs for paged KV-cache attention.

Shared by the tests, the benchmark and the oracle-side checks.  It builds
block tables, slot mappings, copy pairs and N(0,1) values rounded once to the
storage dtype; it computes none of the attention, scatter or copy results.
"""
from .blockmgr import BlockManager, OutOfBlocks  # noqa: F401
from .configs import (CONFIGS, Workload, build_batch, config_workload,  # noqa: F401
                      nan_bits, round_to_dtype, small_workload)

"""Seeded synthetic inputs for the index scorer / top-k (shared by the tests,
the benchmark and the smoke check; holds none of the method's arithmetic)."""
from .gen import (BLOCK, WORKLOADS, DIM, KFMT_BF16, KFMT_NVFP4, Workload, cdiv,
                  config, host_arrays, host_subset, make, round_up)

"""Seeded synthetic inputs for MLA decode over a paged latent cache.

This package draws random numbers and lays them out; it holds none of the
attention arithmetic.  Both the oracle (tests) and the HIP path (tests, bench)
consume exactly the tensors it returns.
"""
from .configs import WORKLOADS, get_workload
from .gen import make_inputs, MlaInputs, quantize_e4m3_blocks

__all__ = ["WORKLOADS", "get_workload", "make_inputs", "MlaInputs", "quantize_e4m3_blocks"]

"""Seeded synthetic inputs shared by the oracle and the GPU path (no method arithmetic)."""
from .gen import (WORKLOADS, Workload, DTYPES, ELEM_BYTES, make_prompt, make_decode,
                  round_to_dtype, sample_heads, unit_vector)

__all__ = ["WORKLOADS", "Workload", "DTYPES", "ELEM_BYTES", "make_prompt", "make_decode",
           "round_to_dtype", "sample_heads", "unit_vector"]

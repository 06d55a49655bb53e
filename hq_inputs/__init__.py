"""Seeded synthetic inputs for the hybrid K4V4/FP16 decode-attention path.

This package only draws numbers: it holds none of the method's arithmetic
(no attention, no quantisation, no selection).  Both the fp64 oracle tests and
the GPU path consume the arrays it returns, so that the two sides are compared
on identical inputs.
"""
from .gen import (WORKLOADS, Workload, workload, sequence, batch, unit_vectors,
                  bf16_round, prefill_queries)

__all__ = ["WORKLOADS", "Workload", "workload", "sequence", "batch",
           "unit_vectors", "bf16_round", "prefill_queries"]

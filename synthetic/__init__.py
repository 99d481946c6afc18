"""Seeded synthetic workloads shared by the tests, the bench and the oracle.

This package holds no step of the attention method: it only describes which
token slots a caller submits (positions, sequence ids, output flags, in
decode-call order), draws the random K/V/Q tensors and draws the optional
free-cell order.  Both the HIP path and the oracle consume what it returns.
"""

from .workloads import (Batch, Workload, QWEN3_06B, tiny, qwen_prefill, cb_decode,
                        mixed, prefix_decode, by_name, WORKLOADS)

__all__ = ["Batch", "Workload", "QWEN3_06B", "tiny", "qwen_prefill", "cb_decode",
           "mixed", "prefix_decode", "by_name", "WORKLOADS"]

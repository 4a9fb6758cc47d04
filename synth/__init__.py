"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle runs.

This module draws random numbers and places them; it holds none of the
cross-entropy arithmetic. Both sides of every parity check receive the same
tensors from here (the oracle gets host copies of them).
"""
from .workloads import WORKLOADS, Inputs, Workload, make_inputs, make_logits, make_targets

__all__ = ["WORKLOADS", "Inputs", "Workload", "make_inputs", "make_logits", "make_targets"]

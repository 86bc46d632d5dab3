"""Seeded synthetic decode-attention inputs (q, K, V, sequence lengths).

This package draws random numbers and plants keys; it holds none of the
attention method's arithmetic.  Both the fp64 oracle and the HIP path are fed
from here, and neither is imported by it.
"""
from .kvgen import WORKLOADS, Workload, make_head, make_case, seq_lens_for, planted_positions

__all__ = ["WORKLOADS", "Workload", "make_head", "make_case", "seq_lens_for", "planted_positions"]

"""Seeded synthetic inputs shared by the tests, the oracle checks and the bench.

Holds no attention or quantisation arithmetic: only draws of lengths, page
placements, tags, reallocations and bf16 K/V/Q values, and the codes,
scales and activations of an INT4 linear layer.
"""
from .configs import (SWEEP_BATCHES, Workload, custom, gqa, in_use_pages, integrity_cost,
                      long_context, mla, sweep, tiny)
from .int4 import Int4Layer, int4_custom, int4_layer

__all__ = ["SWEEP_BATCHES", "Workload", "custom", "gqa", "in_use_pages", "integrity_cost",
           "long_context", "mla", "sweep", "tiny", "Int4Layer", "int4_custom", "int4_layer"]

"""Seeded synthetic workloads for KV-cached grouped-query attention.

This package draws inputs and lays them out in memory; it holds none of the
attention arithmetic. Both the CPU oracle (through the tests and the bench)
and the HIP path consume what it produces, so it is the only code the two
sides share.
"""

from .configs import WORKLOADS, Workload, get_workload
from .synth import (
    Inputs,
    draw_inputs,
    draw_prior_lengths,
    layout_contiguous,
    layout_paged,
    logical_kv,
    make_block_table,
    tree_mask_rows,
    tree_mask_words,
)

__all__ = [
    "WORKLOADS",
    "Workload",
    "get_workload",
    "Inputs",
    "draw_inputs",
    "draw_prior_lengths",
    "layout_contiguous",
    "layout_paged",
    "logical_kv",
    "make_block_table",
    "tree_mask_rows",
    "tree_mask_words",
]

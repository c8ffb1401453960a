"""Seeded synthetic inputs for one context-parallel rank's sparse-attention shard.

This package is the only code shared by the GPU path's tests/benchmark and the
CPU oracle's tests.  It builds inputs and nothing else:

* random draws (``numpy.random.default_rng``) and their round-to-nearest-even
  narrowing to bfloat16, kept as float32 arrays that hold the exact bf16 values;
* the layout arrays that describe which global token each local query row is
  (``q_pos``), which packed sequence it belongs to (``q_seq``) and where the
  packed sequences start (``cu_seqlens``), for contiguous, zigzag and packed
  variable-length (THD) shards.

It contains none of the method's arithmetic: no gating, pooling, selection,
softmax or merge.  The layout follows the context-parallel article ("Context
parallel attention: exchange keys and merge softmax globally", paragraphs on
global positions and on zigzag layouts): a shard keeps global positions, and a
zigzag shard owns two chunks placed symmetrically in the sequence.
"""

from .layout import (
    contiguous_positions,
    zigzag_positions,
    seq_ids_for_positions,
    cu_from_lengths,
)
from .workloads import (
    Workload,
    bf16_round,
    make_workload,
    tiny_block_workload,
    tiny_token_workload,
    up_projection_inputs,
    WORKLOAD_NAMES,
)

__all__ = [
    "contiguous_positions",
    "zigzag_positions",
    "seq_ids_for_positions",
    "cu_from_lengths",
    "Workload",
    "bf16_round",
    "make_workload",
    "tiny_block_workload",
    "tiny_token_workload",
    "up_projection_inputs",
    "WORKLOAD_NAMES",
]

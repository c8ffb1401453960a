"""Permitted keys of a local query row (oracle, fp64 side; test infrastructure).

"Context parallel attention: exchange keys and merge softmax globally", paragraph
on positions and masks: the causal mask is decided by global token positions,
and packed variable-length sequences must not attend across their boundaries.
Megatron-LM issue #4878, "Strategy: allgather CP mode": local queries see the
gathered keys with the causal diagonal shifted to their global offset.

Reading taken: row i may attend to the keys [lo_i, pos_i] (inclusive), where
lo_i is the start of the row's packed sequence.  A row whose sequence id is out
of range, or whose position is not inside its sequence, has no permitted keys.
"""

import numpy as np


def permitted_interval(pos, seq, cu_seqlens):
    """(lo, hi_incl, seq_end) of the keys row (pos, seq) may attend to, or None."""
    n_seq = len(cu_seqlens) - 1
    if seq < 0 or seq >= n_seq:
        return None
    lo, end = int(cu_seqlens[seq]), int(cu_seqlens[seq + 1])
    if pos < lo or pos >= end:
        return None
    return lo, int(pos), end


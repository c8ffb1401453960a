"""Layout arrays for a context-parallel shard (input construction only).

A shard keeps the global token positions of its local query rows; the causal
relation is decided by those global positions, never by local row numbers
(context-parallel article, paragraph on global positions and masks).  Two
placements are built here:

* contiguous: rank r of cp owns global tokens [r*S/cp, (r+1)*S/cp), which is the
  "causal diagonal shifted by cp_rank * local_seq" of Megatron-LM issue #4878
  (section "Strategy: allgather CP mode");
* zigzag: the sequence is cut into 2*cp chunks of S/(2*cp) tokens and rank r
  owns chunks r and 2*cp-1-r, in that physical order (context-parallel
  article, paragraph on zigzag / balanced layouts).

Packed variable-length (THD) streams are described by ``cu_seqlens`` (sequence
start offsets, last entry = total tokens), as in the packed-sequence metadata
of Megatron-LM PR #3674 (Overview and Description).
"""

import numpy as np


def contiguous_positions(global_len: int, cp_size: int, rank: int) -> np.ndarray:
    if global_len % cp_size:
        raise ValueError("global_len must be divisible by cp_size")
    if not 0 <= rank < cp_size:
        raise ValueError("rank out of range")
    local = global_len // cp_size
    return np.arange(rank * local, (rank + 1) * local, dtype=np.int32)


def zigzag_positions(global_len: int, cp_size: int, rank: int) -> np.ndarray:
    if global_len % (2 * cp_size):
        raise ValueError("global_len must be divisible by 2*cp_size")
    if not 0 <= rank < cp_size:
        raise ValueError("rank out of range")
    chunk = global_len // (2 * cp_size)
    first = np.arange(rank * chunk, (rank + 1) * chunk, dtype=np.int32)
    j = 2 * cp_size - 1 - rank
    second = np.arange(j * chunk, (j + 1) * chunk, dtype=np.int32)
    return np.concatenate([first, second])


def cu_from_lengths(lengths) -> np.ndarray:
    lengths = np.asarray(lengths, dtype=np.int64)
    if (lengths < 0).any():
        raise ValueError("negative sequence length")
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    np.cumsum(lengths, out=cu[1:])
    if cu[-1] >= 2**31:
        raise ValueError("packed stream too long for int32 positions")
    return cu.astype(np.int32)


def seq_ids_for_positions(positions, cu_seqlens) -> np.ndarray:
    """Sequence id of each packed position (the sequence whose [start, end) holds it)."""
    positions = np.asarray(positions, dtype=np.int64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    ids = np.searchsorted(cu, positions, side="right") - 1
    return ids.astype(np.int32)

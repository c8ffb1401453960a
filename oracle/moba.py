"""MoBA block gating and top-k block selection (oracle, fp64; test infrastructure).

MoBA issue #34 ("Question on Implementing Context Parallelism with MoBA
Efficient Attention", opening question): each query selects its top-k key
blocks from gating scores computed as Q x K^T, and under context parallelism
the local queries score blocks of the gathered keys.

Readings taken where the page is open (each is listed in the design notes):

* block score = dot product of the query with the mean key of the block,
  unscaled (a positive scale changes neither ranking nor relative margins);
* blocks are cut per packed sequence, starting at the sequence's first token;
  the last block of a sequence may be short and is averaged over its real
  length; blocks never straddle sequences;
* candidates of row i are the blocks of its sequence that end at or before the
  start of its own block (the block holding pos_i); the own block is not ranked
  and is always added;
* ranking is by score descending, ties to the lower block index; if there are
  at most k candidates, all are taken;
* gating is per query head; query head h reads key head h // (Hq / Hkv);
* the output of a row is the global start position of each selected block,
  ascending, padded with -1 to width k + 1.
"""

import numpy as np


def stream_blocks(cu_seqlens, block_size):
    """Blocks of every packed sequence, in stream order.

    Returns (starts, lengths, seq_of_block, first_block_of_seq), where sequence s
    owns blocks first_block_of_seq[s] .. first_block_of_seq[s+1]-1.
    """
    starts, lengths, seqs = [], [], []
    first = [0]
    for s in range(len(cu_seqlens) - 1):
        a, b = int(cu_seqlens[s]), int(cu_seqlens[s + 1])
        t = a
        while t < b:
            starts.append(t)
            lengths.append(min(block_size, b - t))
            seqs.append(s)
            t += block_size
        first.append(len(starts))
    return (np.array(starts, np.int64), np.array(lengths, np.int64),
            np.array(seqs, np.int64), np.array(first, np.int64))


def pool_blocks(k, starts, lengths):
    """Mean key of each block, per key head: mu[b, g, :] (float64)."""
    n_blocks = len(starts)
    mu = np.zeros((n_blocks, k.shape[1], k.shape[2]), dtype=np.float64)
    for b in range(n_blocks):
        s, n = int(starts[b]), int(lengths[b])
        mu[b] = k[s:s + n].astype(np.float64).sum(axis=0) / n
    return mu


def gate_candidates(pos, seq, cu_seqlens, block_size, first_block_of_seq):
    """(own_block, first_candidate, n_candidates) for a row, or None if it has no keys."""
    n_seq = len(cu_seqlens) - 1
    if seq < 0 or seq >= n_seq:
        return None
    lo, end = int(cu_seqlens[seq]), int(cu_seqlens[seq + 1])
    if pos < lo or pos >= end:
        return None
    j_own = (pos - lo) // block_size
    first = int(first_block_of_seq[seq])
    return first + j_own, first, j_own


def gate_scores(q, k, q_pos, q_seq, cu_seqlens, block_size):
    """Gate scores of every row against its candidate blocks.

    Returns a dict with
      scores    [n_q, Hq, max_cand] float64 (NaN past a row's candidate count),
      n_cand    [n_q] candidates per row (-1 for rows without keys),
      first     [n_q] global block index of the first candidate,
      own       [n_q] global block index of the own block (-1 without keys),
      starts    [n_blocks] block start positions.
    """
    starts, lengths, _, first_of_seq = stream_blocks(cu_seqlens, block_size)
    mu = pool_blocks(k, starts, lengths)
    n_q, hq, d = q.shape
    hkv = k.shape[1]
    group = hq // hkv
    info = [gate_candidates(int(p), int(s), cu_seqlens, block_size, first_of_seq)
            for p, s in zip(q_pos, q_seq)]
    max_cand = max([c[2] for c in info if c is not None] + [0])
    scores = np.full((n_q, hq, max(max_cand, 1)), np.nan)
    n_cand = np.full(n_q, -1, np.int64)
    first = np.zeros(n_q, np.int64)
    own = np.full(n_q, -1, np.int64)
    q64 = q.astype(np.float64)
    kv_of_head = np.arange(hq) // group
    for i, c in enumerate(info):
        if c is None:
            continue
        own[i], first[i], n_cand[i] = c
        if n_cand[i] == 0:
            continue
        cand_mu = mu[first[i]:first[i] + n_cand[i]][:, kv_of_head, :]  # [nc, Hq, D]
        scores[i, :, :n_cand[i]] = np.einsum("chd,hd->hc", cand_mu, q64[i])
    return {"scores": scores, "n_cand": n_cand, "first": first, "own": own,
            "starts": starts}


def select_blocks(gate, topk):
    """Top-k blocks per (row, head) plus the own block, as ascending start positions.

    Returns idx [n_q, Hq, topk+1] int32 (-1 padded).
    """
    scores, n_cand = gate["scores"], gate["n_cand"]
    n_q, hq, _ = scores.shape
    starts = gate["starts"]
    idx = np.full((n_q, hq, topk + 1), -1, np.int32)
    for i in range(n_q):
        nc = int(n_cand[i])
        if nc < 0:
            continue
        kept = min(topk, nc)
        # stable sort on the negated score: equal scores keep block order
        order = np.argsort(-scores[i, :, :nc], axis=-1, kind="stable")[:, :kept]
        blocks = np.sort(order, axis=-1) + gate["first"][i]  # [Hq, kept]
        idx[i, :, :kept] = starts[blocks]
        idx[i, :, kept] = starts[gate["own"][i]]
    return idx

"""Brute-force cross-checks for tiny inputs (test infrastructure).

These are deliberately different formulations of what the oracle computes, used
only to pin it:

* ``dense_masked_attention``: one dense softmax over every key of the stream,
  with an explicit multiplicity mask built key by key from the selection
  (a key's weight is its multiplicity times exp(logit)), instead of gathering
  the selected keys;
* ``gate_score_by_keys``: the block score as the mean of the per-key dot
  products (equal to the dot product with the mean key);
* ``topk_by_sort``: top-k by a full Python sort on (-score, index).
"""

import numpy as np


def key_block_start(j, cu_seqlens, block_size):
    """Start of the block (of its own sequence) that holds key j, and that sequence."""
    seq = int(np.searchsorted(cu_seqlens, j, side="right")) - 1
    lo = int(cu_seqlens[seq])
    return lo + ((j - lo) // block_size) * block_size, seq


def multiplicity_mask(mode, idx, q_pos, q_seq, cu_seqlens, hq, block_size=0):
    """C[i, h, j] = how many slots of (i, h) select key j, with the causal/varlen cut."""
    n_q = len(q_pos)
    n_kv = int(cu_seqlens[-1])
    C = np.zeros((n_q, hq, n_kv))
    n_seq = len(cu_seqlens) - 1
    for i in range(n_q):
        pos, seq = int(q_pos[i]), int(q_seq[i])
        if not (0 <= seq < n_seq) or not (cu_seqlens[seq] <= pos < cu_seqlens[seq + 1]):
            continue
        for j in range(n_kv):
            if j > pos:
                break
            if mode == "block":
                bs, kseq = key_block_start(j, cu_seqlens, block_size)
                if kseq != seq:
                    continue
                target = bs
            else:
                if j < cu_seqlens[seq]:
                    continue
                target = j
            for h in range(hq):
                slots = idx[i, 0 if idx.shape[1] == 1 else h]
                C[i, h, j] = np.count_nonzero(np.asarray(slots) == target)
    return C


def dense_masked_attention(q, k, v, C, scale):
    """out[i,h] = sum_j C w_j v_j / sum_j C w_j with w_j = exp(scale q.k_j); 0 if no key."""
    n_q, hq, _ = q.shape
    hkv = k.shape[1]
    group = hq // hkv
    out = np.zeros((n_q, hq, v.shape[2]))
    lse = np.full((n_q, hq), -np.inf)
    for h in range(hq):
        g = h // group
        x = scale * (q[:, h].astype(np.float64) @ k[:, g].astype(np.float64).T)  # [n_q, n_kv]
        with np.errstate(divide="ignore"):
            logc = np.log(C[:, h])
        y = x + logc
        for i in range(n_q):
            if not np.isfinite(y[i]).any():
                continue
            mx = y[i][np.isfinite(y[i])].max()
            e = np.exp(y[i] - mx)
            out[i, h] = e @ v[:, g].astype(np.float64) / e.sum()
            lse[i, h] = mx + np.log(e.sum())
    return out, lse


def gate_score_by_keys(qv, kblock):
    """Mean over the block's keys of q . k."""
    return float(np.mean(kblock.astype(np.float64) @ qv.astype(np.float64)))


def topk_by_sort(scores, k):
    """Indices of the k best scores, ties to the lower index, returned ascending."""
    order = sorted(range(len(scores)), key=lambda j: (-scores[j], j))
    return sorted(order[:k])

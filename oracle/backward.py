"""Gradients of the shard attention with the selection held fixed (oracle, fp64;
test infrastructure).

"Context parallel attention: exchange keys and merge softmax globally",
paragraph on positions and masks: a correct forward does not prove training;
the backward pass must send the gradients of keys and values back to their
owners.  Megatron-LM issue #4878, "Strategy: allgather CP mode", step on the
backward: gradients of the gathered keys and values are computed locally and
then reduce-scattered to the ranks that own them (the reduction across ranks
is out of this one-GPU path; this computes one shard's contribution).

Reading taken: the selection (indices) is a discrete choice and is held fixed;
the loss is L = sum_{i,h} dO[i,h] . O[i,h].  For one (row i, head h) with the
multiset S of selected permitted keys (the forward's definition, a repeated
slot counting its keys again), logits x_j = scale * q . k_j, weights
P_j = exp(x_j - lse) and O = sum_j P_j v_j, the chain rule gives

    dv_j += P_j dO
    dP_j  = dO . v_j
    dx_j  = P_j (dP_j - sum_l P_l dP_l)          (softmax Jacobian)
    dq   += scale sum_j dx_j k_j
    dk_j += scale dx_j q

summed over every occurrence of j in S and over every (row, head) whose
selection holds j; query head h feeds key/value head h // (Hq / Hkv).  A
(row, head) without selected keys contributes nothing.  When the value is the
first Dv columns of the key (absorbed MLA), dk and dv are returned separately
and the gradient of the shared tensor is dk + dv on those columns.
"""

import numpy as np

from .layout import permitted_interval
from .attention import selected_keys, slot_span


def _scatter(dst, mode, slots, interval, block_size, rows):
    """dst[key] += rows[t] for the t-th key of the row's selected multiset.

    Block selections add one slot's span at a time (a span's keys are
    distinct, so a slice add is exact; a repeated slot adds again); token
    selections add by index when their keys are distinct and otherwise use an
    unbuffered add (np.add.at), which adds repeats again.
    """
    if mode == "token":
        keys = selected_keys(mode, slots, interval, block_size)
        if len(np.unique(keys)) == len(keys):
            dst[keys] += rows          # distinct keys: one add each
        else:
            np.add.at(dst, keys, rows)
        return
    lo, hi_incl, seq_end = interval
    t = 0
    for s in slots:
        a, b = slot_span(mode, s, lo, hi_incl, seq_end, block_size)
        dst[a:b] += rows[t:t + (b - a)]
        t += b - a


def shard_backward(q, k, v, q_pos, q_seq, cu_seqlens, mode, idx, scale, dout, block_size=0):
    """(dq [n_q, Hq, Dqk], dk [n_kv, Hkv, Dqk], dv [n_kv, Hkv, Dv]) in float64.

    Arguments as ``shard_forward``; dout [n_q, Hq, Dv] is dL/dO.  Keys, values
    and their gradients are held head-major ([Hkv, n_kv, D]) while they are
    gathered and accumulated.
    """
    n_q, hq, dqk = q.shape
    hkv = k.shape[1]
    group = hq // hkv
    kf = np.ascontiguousarray(np.asarray(k, np.float64).transpose(1, 0, 2))
    vf = np.ascontiguousarray(np.asarray(v, np.float64).transpose(1, 0, 2))
    dq = np.zeros((n_q, hq, dqk))
    dk = np.zeros_like(kf)
    dv = np.zeros_like(vf)
    for i in range(n_q):
        iv = permitted_interval(int(q_pos[i]), int(q_seq[i]), cu_seqlens)
        if idx.shape[1] == 1:
            # one selection for the whole row: each key head's G query heads at once
            keys = selected_keys(mode, idx[i, 0], iv, block_size)
            if len(keys) == 0:
                continue
            for g in range(hkv):
                heads = slice(g * group, (g + 1) * group)
                qm = np.asarray(q[i, heads], np.float64)            # [G, Dqk]
                do = np.asarray(dout[i, heads], np.float64)         # [G, Dv]
                kmat = kf[g][keys]
                vmat = vf[g][keys]
                x = scale * (qm @ kmat.T)                           # [G, n]
                p = np.exp(x - x.max(axis=1, keepdims=True))
                p /= p.sum(axis=1, keepdims=True)
                dp = do @ vmat.T
                dx = p * (dp - (p * dp).sum(axis=1, keepdims=True))
                dq[i, heads] = scale * (dx @ kmat)
                _scatter(dk[g], mode, idx[i, 0], iv, block_size, scale * (dx.T @ qm))
                _scatter(dv[g], mode, idx[i, 0], iv, block_size, p.T @ do)
            continue
        for h in range(hq):
            slots = idx[i, h]
            keys = selected_keys(mode, slots, iv, block_size)
            if len(keys) == 0:
                continue
            g = h // group
            qv = np.asarray(q[i, h], np.float64)
            do = np.asarray(dout[i, h], np.float64)
            kmat = kf[g][keys]
            vmat = vf[g][keys]
            x = scale * (kmat @ qv)
            m = x.max()
            p = np.exp(x - m)
            p /= p.sum()                      # P_j = exp(x_j - lse)
            dp = vmat @ do                    # dP_j
            dx = p * (dp - p @ dp)            # softmax Jacobian
            dq[i, h] = scale * (dx @ kmat)
            _scatter(dk[g], mode, slots, iv, block_size, scale * dx[:, None] * qv[None, :])
            _scatter(dv[g], mode, slots, iv, block_size, p[:, None] * do[None, :])
    return dq, dk.transpose(1, 0, 2), dv.transpose(1, 0, 2)


def loss(q, k, v, q_pos, q_seq, cu_seqlens, mode, idx, scale, dout, block_size=0):
    """L = sum dO . O of the forward (for finite-difference pins)."""
    from .attention import shard_forward
    out, _ = shard_forward(q, k, v, q_pos, q_seq, cu_seqlens, mode, idx, scale, block_size)
    return float((np.asarray(dout, np.float64) * out).sum())

"""Sparse attention over selected chunks, chunk summaries and their merge
(oracle, fp64; test infrastructure).

"Context parallel attention: exchange keys and merge softmax globally":

* paragraph on the chunk summary: a chunk of scores is summarised by its maximum
  m, the denominator l = sum exp(x - m) and the numerator z = sum exp(x - m) v;
  two summaries combine by rescaling both to the larger maximum and adding;
  the division happens only once every contribution is in, and the result is
  the softmax over the union of the chunks;
* paragraph on masking: an all-masked chunk needs a defined neutral summary
  (no -inf minus -inf), and a query with no permitted key needs an explicit
  convention.

Readings taken: the neutral summary is (m, l, z) = (-inf, 0, 0); a query with no
permitted key gets output 0 and log-sum-exp -inf; m and the log-sum-exp are in
natural-log units; logits are x = scale * (q . k).

Since merging summaries reaches exactly the softmax over the selected permitted
keys, ``attend`` / ``attend_spans`` / ``attend_heads`` compute that softmax
directly from its definition (one maximum over all selected keys, one sum).

The selected key set of a (row, head) is the multiset union, over the slots of
its index row, of each slot's permitted keys:

* token slot j: key j if lo_i <= j <= pos_i, else nothing (-1 pads are empty);
* block slot s: the block of the row's sequence that starts at s must be
  aligned to that sequence's block grid (s - lo_i a multiple of the block size)
  and start at or before pos_i; its keys are [s, min(s + B, seq_end)) cut to
  [lo_i, pos_i].  Any other slot value is empty.
Distinct slots are expected (the selectors produce them); a repeated slot
counts its keys again, which is the merge of the same summary twice.
"""

import numpy as np

from .layout import permitted_interval

NEUTRAL_M = -np.inf


def slot_span(mode, s, lo, hi_incl, seq_end, block_size=0):
    """Keys contributed by one index slot, as the range [a, b) (empty when a == b).

    A slot's keys are always consecutive: one token, or one block cut to the
    row's permitted keys.
    """
    s = int(s)
    if s < lo or s > hi_incl:
        return s, s
    if mode == "token":
        return s, s + 1
    if (s - lo) % block_size:
        return s, s
    return s, min(s + block_size, seq_end, hi_incl + 1)


def slot_keys(mode, s, lo, hi_incl, seq_end, block_size=0):
    """Global key positions contributed by one index slot."""
    a, b = slot_span(mode, s, lo, hi_incl, seq_end, block_size)
    return np.arange(a, b, dtype=np.int64)


def selected_keys(mode, slots, interval, block_size=0):
    """Multiset of keys selected by one index row, in slot order."""
    if interval is None:
        return np.zeros(0, np.int64)
    lo, hi_incl, seq_end = interval
    parts = [slot_keys(mode, s, lo, hi_incl, seq_end, block_size) for s in slots]
    return np.concatenate(parts) if parts else np.zeros(0, np.int64)


def attend(qv, kmat, vmat, scale):
    """Softmax attention of one query over the given keys: (o [dv], lse)."""
    if kmat.shape[0] == 0:
        return np.zeros(vmat.shape[1]), -np.inf
    x = scale * (np.asarray(kmat, np.float64) @ np.asarray(qv, np.float64))
    m = x.max()
    e = np.exp(x - m)
    ell = e.sum()
    o = (e @ np.asarray(vmat, np.float64)) / ell
    return o, m + np.log(ell)


def attend_heads(qmat, kmat, vmat, scale):
    """Softmax attention of several queries over one shared key set.

    qmat [nh, Dqk]; returns (o [nh, Dv], lse [nh]).  Each query's softmax is the
    same definition as ``attend``; the logits of all queries are one matrix
    product.  Used where every query head of a row reads the same selection
    (one token-index row per query token).
    """
    nh = qmat.shape[0]
    if kmat.shape[0] == 0:
        return np.zeros((nh, vmat.shape[1])), np.full(nh, -np.inf)
    x = scale * (np.asarray(qmat, np.float64) @ np.asarray(kmat, np.float64).T)  # [nh, n]
    m = x.max(axis=1)
    e = np.exp(x - m[:, None])
    ell = e.sum(axis=1)
    o = (e @ np.asarray(vmat, np.float64)) / ell[:, None]
    return o, m + np.log(ell)


def attend_spans(qv, kg, vg, spans, scale):
    """Softmax attention of one query over the keys of ``spans`` (slot order).

    kg [n_kv, Dqk] and vg [n_kv, Dv] are one key head's keys and values; the
    selected keys are the multiset union of the ranges [a, b) in ``spans``.
    The same definition as ``attend``, with the keys read slot by slot instead
    of gathered: logits of every selected key, their one maximum M, then
    l = sum_j exp(x_j - M) and o = sum_j exp(x_j - M) v_j / l, the sums taken
    slot by slot, key by key.  Returns (o [Dv], lse).
    """
    spans = [(a, b) for a, b in spans if b > a]
    if not spans:
        return np.zeros(vg.shape[1]), -np.inf
    qv = np.asarray(qv, np.float64)
    x = [scale * (np.asarray(kg[a:b], np.float64) @ qv) for a, b in spans]
    m = max(xs.max() for xs in x)
    e = [np.exp(xs - m) for xs in x]
    ell = 0.0
    o = np.zeros(vg.shape[1])
    for es, (a, b) in zip(e, spans):
        ell += es.sum()
        o += es @ np.asarray(vg[a:b], np.float64)
    return o / ell, m + np.log(ell)


def shard_forward(q, k, v, q_pos, q_seq, cu_seqlens, mode, idx, scale, block_size=0,
                  rows=None):
    """Attention output of the shard's rows.

    q [n_q, Hq, Dqk], k [n_kv, Hkv, Dqk], v [n_kv, Hkv, Dv] (any view);
    idx [n_q, idx_heads, W] with idx_heads 1 (shared by all query heads) or Hq.
    Returns (out [n_rows, Hq, Dv] float64, lse [n_rows, Hq] float64).
    """
    if rows is None:
        rows = range(q.shape[0])
    rows = list(rows)
    hq, hkv = q.shape[1], k.shape[1]
    group = hq // hkv
    out = np.zeros((len(rows), hq, v.shape[2]))
    lse = np.full((len(rows), hq), -np.inf)
    for r, i in enumerate(rows):
        iv = permitted_interval(int(q_pos[i]), int(q_seq[i]), cu_seqlens)
        if idx.shape[1] == 1:
            # one selection for the whole row: gather its keys once per key head
            keys = selected_keys(mode, idx[i, 0], iv, block_size)
            for g in range(hkv):
                heads = slice(g * group, (g + 1) * group)
                out[r, heads], lse[r, heads] = attend_heads(q[i, heads], k[keys, g],
                                                            v[keys, g], scale)
            continue
        for h in range(hq):
            g = h // group
            spans = [] if iv is None else [slot_span(mode, sl, *iv, block_size)
                                           for sl in idx[i, h]]
            out[r, h], lse[r, h] = attend_spans(q[i, h], k[:, g], v[:, g], spans, scale)
    return out, lse


def summary(x, vmat):
    """(m, l, z) of a chunk with logits x [n] and values vmat [n, Dv]."""
    x = np.asarray(x, np.float64)
    if x.size == 0:
        return NEUTRAL_M, 0.0, np.zeros(vmat.shape[1])
    m = x.max()
    e = np.exp(x - m)
    return m, e.sum(), e @ np.asarray(vmat, np.float64)


def merge(a, b):
    """Combine two chunk summaries by rescaling both to the larger maximum."""
    ma, la, za = a
    mb, lb, zb = b
    m = max(ma, mb)
    if m == -np.inf:
        return NEUTRAL_M, 0.0, np.zeros_like(np.asarray(za, np.float64))
    wa = 0.0 if ma == -np.inf else np.exp(ma - m)
    wb = 0.0 if mb == -np.inf else np.exp(mb - m)
    return m, wa * la + wb * lb, wa * np.asarray(za, np.float64) + wb * np.asarray(zb, np.float64)


def finalize(s):
    """(o, lse) from a merged summary; zero output and -inf for the neutral one."""
    m, ell, z = s
    if ell <= 0.0 or m == -np.inf:
        return np.zeros_like(np.asarray(z, np.float64)), -np.inf
    return np.asarray(z, np.float64) / ell, m + np.log(ell)


def merge_parts(m, ell, z):
    """Merge P summaries per row in ascending part order.

    m [P, R], ell [P, R], z [P, R, Dv] -> (m [R], ell [R], z [R, Dv]) float64.
    """
    m = np.asarray(m, np.float64)
    ell = np.asarray(ell, np.float64)
    z = np.asarray(z, np.float64)
    n_parts, n_rows = m.shape
    mo = np.full(n_rows, NEUTRAL_M)
    lo = np.zeros(n_rows)
    zo = np.zeros((n_rows, z.shape[2]))
    for r in range(n_rows):
        acc = (NEUTRAL_M, 0.0, np.zeros(z.shape[2]))
        for p in range(n_parts):
            acc = merge(acc, (m[p, r], ell[p, r], z[p, r]))
        mo[r], lo[r], zo[r] = acc
    return mo, lo, zo

"""DSA-style token indexer and top-k token selection (oracle, fp64; test infrastructure).

Megatron-LM PR #3674 ("[1/2] Enable DSA CP, THD with absorbed MLA",
Description): an indexer chooses the top-k key tokens of each query, and sparse
attention then runs over those tokens only.  Megatron-LM issue #4878 ("Strategy:
allgather CP mode"): the indexer runs on the gathered keys and its top-k indices
are in global-sequence coordinates, under the causal mask shifted to the
shard's offset.

Readings taken where the pages are open:

* indexer logit of row i for key j: L[i, j] = sum_h w[i, h] * max(0, iq[i, h] . ik[j])
  with one indexer key per token and per-token, per-head weights, unscaled;
* candidates are the permitted keys [lo_i, pos_i] (the query's own token
  included, not forced);
* ranking is by logit descending, ties to the lower key index; if a row has at
  most k candidates, all are taken;
* the output row is the selected global key positions, ascending, padded with
  -1 to width k.
"""

import numpy as np

from .layout import permitted_interval


def indexer_logits_row(iq_i, ik, w_i, lo, hi_incl):
    """Indexer logits of one row over keys lo..hi_incl (float64 vector)."""
    dots = iq_i.astype(np.float64) @ ik[lo:hi_incl + 1].astype(np.float64).T  # [H_I, n]
    return w_i.astype(np.float64) @ np.maximum(dots, 0.0)


def select_tokens_row(logits, lo, topk):
    """Top-k keys of one row (ascending global positions, -1 padded to topk)."""
    out = np.full(topk, -1, np.int32)
    n = len(logits)
    if n == 0:
        return out
    order = np.argsort(-logits, kind="stable")[:min(topk, n)]
    sel = np.sort(order) + lo
    out[:len(sel)] = sel
    return out


def indexer_topk(iq, ik, w, q_pos, q_seq, cu_seqlens, topk, rows=None):
    """Indexer top-k for the given rows (all rows by default).

    Returns (idx [n_rows, topk] int32, logits list of float64 vectors or None,
    lo list) so callers can examine score margins.
    """
    if rows is None:
        rows = range(len(q_pos))
    rows = list(rows)
    idx = np.full((len(rows), topk), -1, np.int32)
    all_logits, los = [], []
    for r, i in enumerate(rows):
        iv = permitted_interval(int(q_pos[i]), int(q_seq[i]), cu_seqlens)
        if iv is None:
            all_logits.append(None)
            los.append(None)
            continue
        lo, hi_incl, _ = iv
        L = indexer_logits_row(iq[i], ik, w[i], lo, hi_incl)
        idx[r] = select_tokens_row(L, lo, topk)
        all_logits.append(L)
        los.append(lo)
    return idx, all_logits, los

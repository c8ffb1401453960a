"""Absorbed-MLA value up-projection after sparse attention (oracle, fp64;
test infrastructure).

Megatron-LM PR #3674, "[1/2] Enable DSA CP, THD with absorbed MLA":

* the earlier PR's description quoted on that page ("Background"): with matrix
  absorption the key up-projection is folded into the query side and the value
  up-projection is applied after sparse attention;
* the sequence diagram of the review summary: the attention over the latent
  values is followed by an einsum with ``up_v_weight`` that yields
  ``[sq, b, np, v_channels]``.

Reading taken (the pages give the step but not the einsum's subscripts): for
each query head h the latent output o[i, h, :] (width Dl, the value part of the
latent key) is multiplied by that head's value up-projection, a Dv x Dl matrix
stored as a linear layer's weight, rows = output channels:

    out[i, h, d] = sum_c o[i, h, c] * w[h, d, c].
"""

import numpy as np


def v_up_proj(o, w):
    """out [n_q, Hq, Dv] float64 from o [n_q, Hq, Dl] and w [Hq, Dv, Dl]."""
    o = np.asarray(o, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    if o.ndim != 3 or w.ndim != 3 or o.shape[1] != w.shape[0] or o.shape[2] != w.shape[2]:
        raise ValueError("v_up_proj: o [n_q, Hq, Dl] and w [Hq, Dv, Dl] expected")
    out = np.empty((o.shape[0], o.shape[1], w.shape[1]))
    for h in range(o.shape[1]):  # one plain matrix product per head
        out[:, h, :] = o[:, h, :] @ w[h].T
    return out

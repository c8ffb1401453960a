"""Helpers shared by the GPU parity tests: upload of seeded inputs, the index
margin criterion, and the output tolerances.

Tolerances (stated here once and used by every GPU test):
  * selected indices: bit-exact wherever the oracle's k-th vs (k+1)-th score
    margin exceeds 1e-3 relative (ties to the lower index); in near-tie rows
    the GPU must still keep exactly min(k, #candidates) valid indices and
    agree with the oracle on every candidate outside the +-1e-3 band;
  * outputs: 2e-2 max-abs for bf16 inputs, 1e-5 for fp32 inputs, against the
    oracle evaluated on the GPU's own selection.
"""

import numpy as np
import torch

import oracle

REL_MARGIN = 1e-3
TOL = {"bf16": 2e-2, "f32": 1e-5}


def dev_tensor(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x))
    t = t.to("cuda")
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def upload(w):
    """Torch device tensors for a workload (bf16 values are exact)."""
    import context_sparse_attention_amd as csa
    d = {"q": dev_tensor(w.q, w.dtype), "k": dev_tensor(w.k, w.dtype)}
    d["v"] = d["k"][..., : w.dv] if w.v_alias else dev_tensor(w.v, w.dtype)
    if w.mode == "token":
        d["iq"] = dev_tensor(w.iq, w.dtype)
        d["ik"] = dev_tensor(w.ik, w.dtype)
        d["w"] = torch.from_numpy(w.w).to("cuda")
    d["layout"] = csa.Layout(w.q_pos, w.q_seq, w.cu_seqlens)
    return d


def classify_row(scores, gpu_set, ora_set, k):
    """Compare one (row, head) selection with the margin criterion.

    scores: oracle candidate scores (float64) indexed like the candidate ids in
    gpu_set / ora_set (sets of candidate positions 0..n-1).
    Returns "exact", "near_tie_ok" or a failure string.
    """
    n = len(scores)
    kept = min(k, n)
    if len(gpu_set) != kept:
        return f"fail: {len(gpu_set)} kept, {kept} expected"
    if gpu_set == ora_set:
        return "exact"
    if n <= k:
        return "fail: short history must take every candidate"
    srt = np.sort(scores)[::-1]
    sk, sk1 = srt[k - 1], srt[k]
    denom = max(abs(sk), abs(sk1))
    rel = (sk - sk1) / denom if denom > 0 else 0.0
    if rel > REL_MARGIN:
        return f"fail: margin {rel:.2e} but selections differ"
    band = REL_MARGIN * abs(sk)
    for j in gpu_set ^ ora_set:
        if abs(scores[j] - sk) > band:
            return f"fail: candidate {j} (score {scores[j]:.6g}) outside the tie band"
    return "near_tie_ok"


def check_moba_indices(w, gpu_idx, gate=None):
    """Counts per category for a MoBA selection; raises on any failure."""
    if gate is None:
        gate = oracle.gate_scores(w.q, w.k, w.q_pos, w.q_seq, w.cu_seqlens, w.block_size)
    ora_idx = oracle.select_blocks(gate, w.topk)
    starts = gate["starts"]
    counts = {"exact": 0, "near_tie_ok": 0, "no_keys": 0}
    fails = []
    for i in range(w.n_q):
        nc = int(gate["n_cand"][i])
        if nc < 0:
            assert (gpu_idx[i] == -1).all(), f"row {i} has no keys but selects"
            counts["no_keys"] += 1
            continue
        first = int(gate["first"][i])
        own_start = int(starts[gate["own"][i]])
        for h in range(w.hq):
            row = gpu_idx[i, h]
            valid = row[row >= 0]
            if len(valid) == 0 or valid[-1] != own_start:
                fails.append((i, h, "own block missing"))
                continue
            if (row[len(valid):] != -1).any() or (np.diff(valid) <= 0).any():
                fails.append((i, h, "not ascending / padded"))
                continue
            gpu_c = set(int(np.searchsorted(starts, s)) - first for s in valid[:-1])
            if any(c < 0 or c >= nc for c in gpu_c):
                fails.append((i, h, "selected a block that is not a candidate"))
                continue
            ora_row = ora_idx[i, h]
            ora_c = set(int(np.searchsorted(starts, s)) - first for s in ora_row[ora_row >= 0][:-1])
            res = classify_row(gate["scores"][i, h, :nc], gpu_c, ora_c, w.topk)
            if res.startswith("fail"):
                fails.append((i, h, res))
            else:
                counts[res] += 1
    assert not fails, f"{len(fails)} index failures, first: {fails[:5]}"
    return counts


def check_token_indices(w, rows, gpu_idx_rows):
    """Margin criterion for DSA rows; gpu_idx_rows [len(rows), topk]."""
    ora_idx, logits, los = oracle.indexer_topk(w.iq, w.ik, w.w, w.q_pos, w.q_seq,
                                               w.cu_seqlens, w.topk, rows=rows)
    counts = {"exact": 0, "near_tie_ok": 0, "no_keys": 0}
    fails = []
    for r, i in enumerate(rows):
        row = gpu_idx_rows[r]
        if logits[r] is None:
            assert (row == -1).all()
            counts["no_keys"] += 1
            continue
        valid = row[row >= 0]
        if (row[len(valid):] != -1).any() or (np.diff(valid) <= 0).any():
            fails.append((i, "not ascending / padded"))
            continue
        lo = los[r]
        gpu_c = set((valid - lo).tolist())
        ora = ora_idx[r]
        ora_c = set((ora[ora >= 0] - lo).tolist())
        res = classify_row(logits[r], gpu_c, ora_c, w.topk)
        if res.startswith("fail"):
            fails.append((i, res))
        else:
            counts[res] += 1
    assert not fails, f"{len(fails)} index failures, first: {fails[:5]}"
    return counts


def sample_rows(n_q, count, seed=0, must=()):
    rng = np.random.default_rng(seed)
    rows = set(int(x) for x in must if 0 <= x < n_q)
    rows |= set(rng.choice(n_q, size=min(count, n_q), replace=False).tolist())
    return sorted(rows)

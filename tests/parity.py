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
from oracle_pool import classify_row, REL_MARGIN  # noqa: F401

TOL = {"bf16": 2e-2, "f32": 1e-5}
# relative bound on the gate's fp32 block scores: the block mean is summed in
# fp32 and split into two bf16 parts (~2^-17), and the dot product is an fp32
# sum of D products; 5e-5 of sum_d |q_d| mean_t |k_td| covers both
GATE_SCORE_REL = 5e-5
# relative bound on the indexer's fp32 logits (exact bf16 products, fp32 sums
# over D_I and over the heads), of sum_h w_h sum_d |iq_hd| |ik_jd|
INDEXER_SCORE_REL = 5e-5
SENTINEL = -7777  # pre-filled into index outputs: every element must be overwritten


def poisoned(shape, dtype):
    """A device tensor pre-filled with NaN (floating point) or SENTINEL (int32)."""
    if dtype == torch.int32:
        return torch.full(shape, SENTINEL, dtype=dtype, device="cuda")
    return torch.full(shape, float("nan"), dtype=dtype, device="cuda")


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


def check_moba_scores(w, gate, gpu_idx, gpu_score):
    """The gate's score output: +inf for the own block, -inf for padding, and for
    each selected candidate block the oracle's score within GATE_SCORE_REL of
    sum_d |q_d| mean_t |k_td| (the block's mean absolute key).  Returns the
    worst absolute error and the number of scores compared."""
    starts = gate["starts"]
    _, lengths, _, _ = oracle.stream_blocks(w.cu_seqlens, w.block_size)
    absmean = oracle.pool_blocks(np.abs(w.k), starts, lengths)  # [n_blocks, Hkv, D]
    group = w.hq // w.hkv
    kv = np.arange(w.hq) // group
    worst, n = 0.0, 0
    for i in range(w.n_q):
        row, sc = gpu_idx[i], gpu_score[i]
        pad = row == -1
        assert np.isneginf(sc[pad]).all(), f"row {i}: padding scores are not -inf"
        if gate["n_cand"][i] < 0:
            continue
        own = row == int(starts[gate["own"][i]])
        assert np.isposinf(sc[own]).all(), f"row {i}: own-block scores are not +inf"
        sel = ~pad & ~own
        if not sel.any():
            continue
        h_of, s_of = np.nonzero(sel)
        blk = np.searchsorted(starts, row[sel])
        c = blk - int(gate["first"][i])
        ref = gate["scores"][i, h_of, c]
        a = (np.abs(w.q[i, h_of].astype(np.float64)) *
             absmean[blk, kv[h_of]]).sum(axis=-1)
        err = np.abs(sc[sel].astype(np.float64) - ref)
        bad = err > GATE_SCORE_REL * a
        assert not bad.any(), (f"row {i} head {h_of[bad][0]}: gate score error "
                               f"{err[bad][0]:.3e} > {GATE_SCORE_REL * a[bad][0]:.3e}")
        worst = max(worst, float(err.max()))
        n += int(sel.sum())
    return worst, n


def sample_rows(n_q, count, seed=0, must=()):
    rng = np.random.default_rng(seed)
    rows = set(int(x) for x in must if 0 <= x < n_q)
    rows |= set(rng.choice(n_q, size=min(count, n_q), replace=False).tolist())
    return sorted(rows)

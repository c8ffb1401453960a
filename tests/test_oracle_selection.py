"""Pins for the oracle's MoBA block gating and DSA token indexer selection (CPU only).

Block selection follows MoBA issue #34 (gating scores Q x K^T, top-k blocks);
token selection follows Megatron-LM PR #3674 (an indexer picks the top-k keys of
each query) and issue #4878 (indices in global coordinates, causal offset).
The pins: a brute-force gate (mean of per-key products), a brute-force indexer
(explicit loops over heads and dimensions), a full Python sort for top-k,
closed-form ties and a planted winning block.
"""

import numpy as np
import pytest

import oracle
from oracle import brute
from csa_inputs import tiny_block_workload, tiny_token_workload


def _brute_gate_idx(w):
    """Block selection written from scratch with the brute-force helpers."""
    hq, hkv = w.hq, w.hkv
    idx = np.full((w.n_q, hq, w.topk + 1), -1, np.int32)
    cu = w.cu_seqlens
    for i in range(w.n_q):
        pos, seq = int(w.q_pos[i]), int(w.q_seq[i])
        lo, end = int(cu[seq]), int(cu[seq + 1])
        own_start = lo + ((pos - lo) // w.block_size) * w.block_size
        cand_starts = list(range(lo, own_start, w.block_size))
        for h in range(hq):
            g = h // (hq // hkv)
            scores = [brute.gate_score_by_keys(w.q[i, h], w.k[s:min(s + w.block_size, end), g])
                      for s in cand_starts]
            chosen = [cand_starts[j] for j in brute.topk_by_sort(scores, w.topk)]
            row = sorted(chosen) + [own_start]
            idx[i, h, :len(row)] = row
    return idx


@pytest.mark.parametrize("seed,lengths,topk,block,layout", [
    (0, (40, 24), 2, 8, "contiguous"),
    (1, (64,), 3, 8, "zigzag"),
    (2, (13, 30, 21), 1, 4, "all"),
    (3, (77, 51), 5, 8, "all"),
])
def test_gate_selection_matches_bruteforce(seed, lengths, topk, block, layout):
    w = tiny_block_workload(seed=seed, lengths=lengths, topk=topk, block=block,
                            layout=layout)
    gate = oracle.gate_scores(w.q, w.k, w.q_pos, w.q_seq, w.cu_seqlens, w.block_size)
    idx = oracle.select_blocks(gate, w.topk)
    np.testing.assert_array_equal(idx, _brute_gate_idx(w))


def test_gate_identity_mean_key_equals_mean_of_products():
    w = tiny_block_workload(seed=5, lengths=(64, 40), topk=2, layout="all")
    gate = oracle.gate_scores(w.q, w.k, w.q_pos, w.q_seq, w.cu_seqlens, w.block_size)
    starts = gate["starts"]
    checked = 0
    for i in range(w.n_q):
        nc = gate["n_cand"][i]
        for h in range(w.hq):
            g = h // (w.hq // w.hkv)
            for c in range(nc):
                s = int(starts[gate["first"][i] + c])
                ref = brute.gate_score_by_keys(w.q[i, h], w.k[s:s + w.block_size, g])
                assert gate["scores"][i, h, c] == pytest.approx(ref, rel=1e-12, abs=1e-13)
                checked += 1
    assert checked > 100


def test_gate_ties_all_zero_keys_pick_lowest_blocks():
    w = tiny_block_workload(seed=6, lengths=(64,), topk=3, layout="all")
    w.k = np.zeros_like(w.k)
    gate = oracle.gate_scores(w.q, w.k, w.q_pos, w.q_seq, w.cu_seqlens, w.block_size)
    idx = oracle.select_blocks(gate, w.topk)
    for i in range(w.n_q):
        own = (int(w.q_pos[i]) // w.block_size) * w.block_size
        expect = list(range(0, min(own, 3 * w.block_size), w.block_size)) + [own]
        for h in range(w.hq):
            row = [x for x in idx[i, h] if x >= 0]
            assert row == expect


def test_gate_planted_block_is_selected():
    w = tiny_block_workload(seed=7, lengths=(64,), topk=1, layout="all", d=8)
    w.q = np.ones_like(w.q)
    k = w.k.copy()
    k[16:24] += 5.0  # block starting at 16, every key component +5
    w.k = k
    gate = oracle.gate_scores(w.q, w.k, w.q_pos, w.q_seq, w.cu_seqlens, w.block_size)
    idx = oracle.select_blocks(gate, w.topk)
    for i in range(w.n_q):
        if w.q_pos[i] >= 24 + 8:  # block 16..23 is a candidate once the own block starts >= 24
            assert 16 in idx[i, 0]


def test_gate_short_histories_take_every_candidate():
    w = tiny_block_workload(seed=8, lengths=(40,), topk=8, layout="all")
    gate = oracle.gate_scores(w.q, w.k, w.q_pos, w.q_seq, w.cu_seqlens, w.block_size)
    idx = oracle.select_blocks(gate, w.topk)
    for i in range(w.n_q):
        own = (int(w.q_pos[i]) // w.block_size) * w.block_size
        assert [x for x in idx[i, 0] if x >= 0] == list(range(0, own + 1, w.block_size))


def _brute_indexer_logits(iq_i, ik, w_i, lo, hi_incl):
    out = []
    for j in range(lo, hi_incl + 1):
        total = 0.0
        for h in range(iq_i.shape[0]):
            dot = 0.0
            for d in range(iq_i.shape[1]):
                dot += float(iq_i[h, d]) * float(ik[j, d])
            total += float(w_i[h]) * max(0.0, dot)
        out.append(total)
    return np.array(out)


@pytest.mark.parametrize("seed,lengths,topk", [(0, (48, 16), 5), (1, (30, 34), 40),
                                               (2, (9, 9, 9), 3)])
def test_indexer_matches_bruteforce(seed, lengths, topk):
    w = tiny_token_workload(seed=seed, lengths=lengths, topk=topk)
    idx, logits, los = oracle.indexer_topk(w.iq, w.ik, w.w, w.q_pos, w.q_seq,
                                           w.cu_seqlens, w.topk)
    for i in range(w.n_q):
        lo = int(w.cu_seqlens[w.q_seq[i]])
        ref = _brute_indexer_logits(w.iq[i], w.ik, w.w[i], lo, int(w.q_pos[i]))
        np.testing.assert_allclose(logits[i], ref, rtol=1e-12, atol=1e-12)
        expect = [lo + j for j in brute.topk_by_sort(list(ref), topk)]
        row = [x for x in idx[i] if x >= 0]
        assert row == expect
        assert (idx[i, len(row):] == -1).all()


def test_indexer_ties_pick_lowest_tokens():
    w = tiny_token_workload(seed=3, lengths=(40, 24), topk=6)
    w.iq = -np.ones_like(w.iq)
    w.ik = np.ones_like(w.ik)  # every product negative, every logit ReLU(.) = 0
    idx, logits, _ = oracle.indexer_topk(w.iq, w.ik, w.w, w.q_pos, w.q_seq, w.cu_seqlens,
                                         w.topk)
    for i in range(w.n_q):
        lo = int(w.cu_seqlens[w.q_seq[i]])
        n = int(w.q_pos[i]) - lo + 1
        assert not logits[i].any()
        expect = list(range(lo, lo + min(n, w.topk)))
        assert [x for x in idx[i] if x >= 0] == expect


def test_indexer_single_head_unit_weight_is_plain_dot_ranking():
    w = tiny_token_workload(seed=4, lengths=(64,), hi=1, topk=7)
    w.w = np.ones_like(w.w)
    w.ik = np.abs(w.ik)
    w.iq = np.abs(w.iq)  # positive products: ReLU is the identity
    idx, _, _ = oracle.indexer_topk(w.iq, w.ik, w.w, w.q_pos, w.q_seq, w.cu_seqlens, w.topk)
    for i in range(w.n_q):
        p = int(w.q_pos[i])
        dots = w.ik[: p + 1].astype(np.float64) @ w.iq[i, 0].astype(np.float64)
        expect = sorted(np.argsort(-dots, kind="stable")[: w.topk].tolist())
        assert [x for x in idx[i] if x >= 0] == expect


def test_indexer_rows_without_keys_are_all_pads():
    w = tiny_token_workload(seed=5, lengths=(30, 34), topk=4)
    q_seq = w.q_seq.copy()
    q_seq[2] = 1  # sequence 1 starts after position 2
    idx, logits, _ = oracle.indexer_topk(w.iq, w.ik, w.w, w.q_pos, q_seq, w.cu_seqlens,
                                         w.topk)
    assert (idx[2] == -1).all() and logits[2] is None

"""Pins for the oracle's sparse shard attention (CPU only).

Each test ties ``oracle.shard_forward`` to something other than itself: a dense
brute-force softmax with an explicit mask, torch's scaled_dot_product_attention
(CPU, float64) on the dense special case, the slice-of-a-full-run check of
Megatron-LM issue #4878 (planned single-GPU test: the shard output at the
causal offset equals the matching slice of a full single-rank run), packing
invariance for THD streams, the GQA / aliased-value reductions, the no-key
convention and softmax invariants.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
from csa_inputs import (tiny_block_workload, tiny_token_workload, make_workload,
                        contiguous_positions, zigzag_positions, seq_ids_for_positions)


def _moba_idx(w):
    gate = oracle.gate_scores(w.q, w.k, w.q_pos, w.q_seq, w.cu_seqlens, w.block_size)
    return oracle.select_blocks(gate, w.topk)


def _run(w, idx, rows=None, q=None, k=None, v=None, q_pos=None, q_seq=None, cu=None):
    return oracle.shard_forward(
        w.q if q is None else q, w.k if k is None else k, w.value if v is None else v,
        w.q_pos if q_pos is None else q_pos, w.q_seq if q_seq is None else q_seq,
        w.cu_seqlens if cu is None else cu, w.mode, idx, w.scale, w.block_size, rows)


@pytest.mark.parametrize("seed,layout,lengths,topk", [
    (0, "contiguous", (40, 24), 2),
    (1, "zigzag", (64,), 3),
    (2, "all", (13, 30, 21), 1),
    (3, "all", (64,), 0),
])
def test_block_mode_matches_dense_masked_bruteforce(seed, layout, lengths, topk):
    w = tiny_block_workload(seed=seed, layout=layout, lengths=lengths, topk=topk)
    idx = _moba_idx(w)
    out, lse = _run(w, idx)
    C = brute.multiplicity_mask("block", idx, w.q_pos, w.q_seq, w.cu_seqlens, w.hq,
                                w.block_size)
    ref, ref_lse = brute.dense_masked_attention(w.q, w.k, w.value, C, w.scale)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-13)


def test_block_mode_arbitrary_slots_match_bruteforce():
    """Caller-made index rows: pads, misaligned, future, other-sequence and repeated slots."""
    w = tiny_block_workload(seed=4, layout="all", lengths=(20, 28, 16), topk=2)
    rng = np.random.default_rng(4)
    W = 6
    idx = rng.integers(-3, w.n_kv + 3, size=(w.n_q, w.hq, W)).astype(np.int32)
    # make a good share of slots aligned block starts of the row's own sequence
    for i in range(w.n_q):
        lo = int(w.cu_seqlens[w.q_seq[i]])
        for h in range(w.hq):
            for s in range(0, W, 2):
                idx[i, h, s] = lo + w.block_size * int(rng.integers(0, 4))
    idx[::3, :, 1] = idx[::3, :, 0]  # repeated slot
    out, lse = _run(w, idx)
    C = brute.multiplicity_mask("block", idx, w.q_pos, w.q_seq, w.cu_seqlens, w.hq,
                                w.block_size)
    ref, ref_lse = brute.dense_masked_attention(w.q, w.k, w.value, C, w.scale)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("seed,shared", [(0, True), (1, False)])
def test_token_mode_matches_dense_masked_bruteforce(seed, shared):
    w = tiny_token_workload(seed=seed)
    rng = np.random.default_rng(seed)
    heads = 1 if shared else w.hq
    idx = rng.integers(-2, w.n_kv + 2, size=(w.n_q, heads, 7)).astype(np.int32)
    out, lse = _run(w, idx)
    C = brute.multiplicity_mask("token", idx, w.q_pos, w.q_seq, w.cu_seqlens, w.hq)
    ref, ref_lse = brute.dense_masked_attention(w.q, w.k, w.value, C, w.scale)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-13)


def test_token_mode_with_indexer_selection_matches_bruteforce():
    w = tiny_token_workload(seed=5)
    idx, _, _ = oracle.indexer_topk(w.iq, w.ik, w.w, w.q_pos, w.q_seq, w.cu_seqlens, w.topk)
    idx = idx[:, None, :]
    out, lse = _run(w, idx)
    C = brute.multiplicity_mask("token", idx, w.q_pos, w.q_seq, w.cu_seqlens, w.hq)
    ref, ref_lse = brute.dense_masked_attention(w.q, w.k, w.value, C, w.scale)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)


def _sdpa_dense_causal(q, k, v, scale, seq_lengths):
    """torch SDPA (float64, CPU) over the packed stream with a block-diagonal causal mask."""
    n = q.shape[0]
    seq = np.repeat(np.arange(len(seq_lengths)), seq_lengths)
    allowed = (np.arange(n)[None, :] <= np.arange(n)[:, None]) & (seq[:, None] == seq[None, :])
    hq, hkv = q.shape[1], k.shape[1]
    kk = np.repeat(k, hq // hkv, axis=1)
    vv = np.repeat(v, hq // hkv, axis=1)
    tq = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2)
    tk = torch.from_numpy(kk.astype(np.float64)).permute(1, 0, 2)
    tv = torch.from_numpy(vv.astype(np.float64)).permute(1, 0, 2)
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=torch.from_numpy(allowed), scale=scale)
    return out.permute(1, 0, 2).numpy()


def test_dense_special_case_matches_torch_sdpa():
    """With k at least the number of blocks, block selection is dense causal attention."""
    lengths = (37, 27)
    total = sum(lengths)
    rng = np.random.default_rng(7)
    q_all = rng.standard_normal((total, 4, 8))
    w = tiny_block_workload(seed=7, layout="all", lengths=lengths, topk=16)
    w.q = q_all
    idx = _moba_idx(w)
    out, _ = _run(w, idx)
    ref = _sdpa_dense_causal(q_all, w.k, w.value, w.scale, lengths)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_dense_f32_workload_is_dense_causal():
    """The 512-token fp32 workload (top-8 of 64-token blocks) equals dense causal SDPA."""
    w = make_workload("dense_f32")
    idx = _moba_idx(w)
    out, _ = _run(w, idx)
    rng = np.random.default_rng(1)
    q_full = rng.standard_normal(size=(512, 2, 64), dtype=np.float32)  # same first draw
    np.testing.assert_array_equal(q_full[w.q_pos], w.q)
    ref = _sdpa_dense_causal(q_full, w.k, w.value, w.scale, [512])[w.q_pos]
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("layout", ["contiguous", "zigzag"])
def test_shard_rows_equal_full_run_slice_bitwise(layout):
    """Every rank's shard, stitched, equals the single-rank full run bit for bit."""
    total, cp = 64, 4
    full = tiny_block_workload(seed=8, layout="all", lengths=(total,), topk=2, hq=2,
                               hkv=1, d=8, block=8)
    idx_full = _moba_idx(full)
    out_full, lse_full = _run(full, idx_full)
    covered = np.zeros(total, int)
    for rank in range(cp):
        pos = (contiguous_positions if layout == "contiguous" else zigzag_positions)(
            total, cp, rank)
        q_seq = seq_ids_for_positions(pos, full.cu_seqlens)
        q_loc = full.q[pos]
        gate = oracle.gate_scores(q_loc, full.k, pos, q_seq, full.cu_seqlens,
                                  full.block_size)
        idx = oracle.select_blocks(gate, full.topk)
        np.testing.assert_array_equal(idx, idx_full[pos])
        out, lse = _run(full, idx, q=q_loc, q_pos=pos, q_seq=q_seq)
        assert np.array_equal(out, out_full[pos])
        assert np.array_equal(lse, lse_full[pos])
        covered[pos] += 1
    assert (covered == 1).all()


def test_thd_packing_invariance():
    """A packed row equals the same sequence run alone; other sequences' keys do not matter."""
    lengths = (24, 40, 17)
    w = tiny_block_workload(seed=9, layout="all", lengths=lengths, topk=2)
    idx = _moba_idx(w)
    out, lse = _run(w, idx)
    cu = w.cu_seqlens
    for s in range(len(lengths)):
        a, b = int(cu[s]), int(cu[s + 1])
        rows = np.arange(a, b)
        alone_cu = np.array([0, b - a], np.int32)
        pos = (rows - a).astype(np.int32)
        q_seq = np.zeros(len(rows), np.int32)
        gate = oracle.gate_scores(w.q[rows], w.k[a:b], pos, q_seq, alone_cu, w.block_size)
        idx_alone = oracle.select_blocks(gate, w.topk)
        np.testing.assert_array_equal(np.where(idx[rows] >= 0, idx[rows] - a, -1), idx_alone)
        out_a, lse_a = oracle.shard_forward(w.q[rows], w.k[a:b], w.value[a:b], pos, q_seq,
                                            alone_cu, "block", idx_alone, w.scale,
                                            w.block_size)
        np.testing.assert_allclose(out[rows], out_a, rtol=1e-13, atol=1e-14)
    # perturbing the keys and values of the other sequences changes nothing in sequence 1
    k2, v2 = w.k.copy(), w.value.copy()
    k2[: cu[1]] += 5.0
    v2[cu[2]:] -= 3.0
    rows1 = np.arange(cu[1], cu[2])
    out2, _ = _run(w, idx, k=k2, v=v2)
    assert np.array_equal(out2[rows1], out[rows1])


def test_gqa_equals_mha_with_repeated_heads():
    w = tiny_block_workload(seed=10, layout="all", lengths=(48,), hq=4, hkv=2, topk=2)
    idx = _moba_idx(w)
    out, lse = _run(w, idx)
    k_rep = np.repeat(w.k, 2, axis=1)
    v_rep = np.repeat(w.value, 2, axis=1)
    out2, lse2 = _run(w, idx, k=k_rep, v=v_rep)
    np.testing.assert_allclose(out, out2, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(lse, lse2, rtol=1e-14, atol=1e-15)


def test_aliased_value_equals_copied_value():
    w = tiny_token_workload(seed=11)
    idx, _, _ = oracle.indexer_topk(w.iq, w.ik, w.w, w.q_pos, w.q_seq, w.cu_seqlens, w.topk)
    idx = idx[:, None, :]
    alias = w.k[..., : w.dv]
    assert np.shares_memory(alias, w.k)
    out_a, _ = _run(w, idx, v=alias)
    out_c, _ = _run(w, idx, v=np.ascontiguousarray(alias.copy()))
    assert np.array_equal(out_a, out_c)


def test_rows_without_keys_are_zero_and_never_nan():
    w = tiny_block_workload(seed=12, layout="all", lengths=(20, 20), topk=2)
    idx = _moba_idx(w)
    q_pos = w.q_pos.copy()
    q_seq = w.q_seq.copy()
    q_seq[3] = 1          # sequence 1 starts at 20 > position 3
    q_seq[25] = 7         # no such sequence
    q_pos[30] = 40        # beyond the stream
    out, lse = _run(w, idx, q_pos=q_pos, q_seq=q_seq)
    for r in (3, 25, 30):
        assert not out[r].any() and (lse[r] == -np.inf).all()
    assert not np.isnan(out).any() and not np.isnan(lse).any()
    # all-masked index rows: only pads / future slots
    idx2 = np.full_like(idx, -1)
    idx2[:, :, 0] = w.n_kv - 1
    out2, lse2 = _run(w, idx2)
    assert not np.isnan(out2).any()
    assert (lse2[: w.n_q - 1] == -np.inf).all()


def test_softmax_invariants():
    w = tiny_block_workload(seed=13, layout="all", lengths=(56,), topk=3)
    idx = _moba_idx(w)
    v_const = np.full_like(w.value, 2.5)
    out, _ = _run(w, idx, v=v_const)
    np.testing.assert_allclose(out, 2.5, rtol=0, atol=1e-14)
    out, _ = _run(w, idx)
    for i in range(w.n_q):
        iv = oracle.permitted_interval(int(w.q_pos[i]), int(w.q_seq[i]), w.cu_seqlens)
        for h in range(w.hq):
            keys = oracle.selected_keys("block", idx[i, h], iv, w.block_size)
            vals = w.value[keys, h // (w.hq // w.hkv)]
            assert (out[i, h] >= vals.min(axis=0) - 1e-12).all()
            assert (out[i, h] <= vals.max(axis=0) + 1e-12).all()
    # reordering the slots of each row only changes rounding
    out_rev, _ = _run(w, idx[:, :, ::-1].copy())
    np.testing.assert_allclose(out_rev, out, rtol=1e-13, atol=1e-14)


def test_planted_transposed_operand_is_caught():
    """An attend() that uses the value's heads the wrong way round fails the brute-force pin."""
    w = tiny_block_workload(seed=14, layout="all", lengths=(32,), hq=2, hkv=2, topk=2)
    idx = _moba_idx(w)
    C = brute.multiplicity_mask("block", idx, w.q_pos, w.q_seq, w.cu_seqlens, w.hq,
                                w.block_size)
    ref, _ = brute.dense_masked_attention(w.q, w.k, w.value, C, w.scale)
    v_swapped = w.value[:, ::-1].copy()
    out, _ = _run(w, idx, v=v_swapped)
    assert not np.allclose(out, ref, rtol=1e-6, atol=1e-6)

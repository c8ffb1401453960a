"""GPU parity: every C-ABI entry point against the fp64 oracle (MI355X only).

Inputs are the seeded workloads of ``csa_inputs``; the oracle reads the same
values.  Index outputs follow the margin criterion and outputs the tolerances
of tests/parity.py.  Small cases check every row; the five named workloads run
at full size in the launch configuration the benchmark uses and check every
selection (MoBA) or sampled rows (DSA indexer, attention outputs).
"""

import numpy as np
import pytest
import torch

import oracle
from csa_inputs import make_workload, tiny_block_workload, tiny_token_workload
from parity import (TOL, upload, check_moba_indices, check_token_indices, sample_rows,
                    dev_tensor)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

if torch.cuda.is_available():
    import context_sparse_attention_amd as csa


def _say(*a):
    print("[case]", *a, flush=True)


def _attn(w, d, idx, out_dtype=None, mode=None):
    mode = (csa.CSA_SEL_BLOCK if w.mode == "block" else csa.CSA_SEL_TOKEN) if mode is None else mode
    out, lse = csa.sparse_attn_fwd_shard(d["q"], d["k"], d["v"], d["layout"], mode, idx,
                                         block_size=w.block_size, softmax_scale=w.scale,
                                         out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


def _check_out(w, idx_np, out, lse, rows, tol):
    ref, ref_lse = oracle.shard_forward(w.q, w.k, w.value, w.q_pos, w.q_seq, w.cu_seqlens,
                                        w.mode, idx_np, w.scale, w.block_size, rows=rows)
    got = out[rows]
    assert not np.isnan(got).any() and not np.isnan(lse[rows]).any()
    err = np.abs(got - ref).max() if got.size else 0.0
    assert err <= tol, f"max abs error {err:.3e} > {tol}"
    fin = np.isfinite(ref_lse)
    assert (np.isfinite(lse[rows]) == fin).all()
    if fin.any():
        lerr = np.abs(lse[rows][fin] - ref_lse[fin]).max()
        assert lerr <= max(tol, 1e-4), f"lse error {lerr:.3e}"
    return err


# bf16 cases with D in {64, 128} and blocks of a multiple of 64 run the MFMA path;
# the others (and every fp32 case) run the general-shape path.
TINY_BLOCK = [
    dict(seed=0, lengths=(200, 120), layout="contiguous", cp=2, rank=1, hq=4, hkv=2, d=64,
         block=64, topk=2),
    dict(seed=1, lengths=(512,), layout="zigzag", cp=4, rank=1, hq=8, hkv=2, d=128, block=64,
         topk=3),
    dict(seed=2, lengths=(77, 300, 19, 116), layout="all", hq=4, hkv=4, d=128, block=64,
         topk=4),
    dict(seed=3, lengths=(640,), layout="contiguous", cp=4, rank=3, hq=2, hkv=1, d=64,
         block=64, topk=1),
    dict(seed=5, lengths=(333, 700, 91), layout="all", hq=16, hkv=2, d=128, block=128,
         topk=2),
    dict(seed=6, lengths=(300, 212), layout="all", hq=4, hkv=2, d=64, block=48, topk=3),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", range(len(TINY_BLOCK)))
def test_tiny_block_gate_and_attention(case, dtype):
    w = tiny_block_workload(dtype=dtype, **TINY_BLOCK[case])
    _say("tiny block", case, dtype, w.q.shape, w.k.shape)
    d = upload(w)
    idx = csa.moba_gate_topk(d["q"], d["k"], d["layout"], w.block_size, w.topk)
    torch.cuda.synchronize()
    idx_np = idx.cpu().numpy()
    counts = check_moba_indices(w, idx_np)
    assert counts["exact"] > 0
    for out_dtype in (torch.float32, d["q"].dtype):
        out, lse = _attn(w, d, idx, out_dtype=out_dtype)
        tol = TOL[dtype] if out_dtype == torch.float32 else TOL["bf16"]
        _check_out(w, idx_np, out, lse, list(range(w.n_q)), tol)


@pytest.mark.parametrize("dtype,block", [("f32", 16), ("bf16", 16), ("bf16", 64)])
def test_tiny_block_arbitrary_slots(dtype, block):
    """Caller-made index rows: pads, misaligned, out-of-range, future and repeated slots."""
    w = tiny_block_workload(seed=4, layout="all", lengths=(300, 420, 180), hq=4, hkv=2, d=64,
                            block=block, topk=2, dtype=dtype)
    _say("arbitrary slots", dtype, block)
    rng = np.random.default_rng(4)
    W = 7
    idx = rng.integers(-3, w.n_kv + 3, size=(w.n_q, w.hq, W)).astype(np.int32)
    for i in range(w.n_q):
        lo = int(w.cu_seqlens[w.q_seq[i]])
        for s in range(0, W, 2):
            idx[i, :, s] = lo + w.block_size * rng.integers(0, 8, size=w.hq)
    idx[::3, :, 1] = idx[::3, :, 0]
    d = upload(w)
    out, lse = _attn(w, d, torch.from_numpy(idx).cuda(), out_dtype=torch.float32)
    _check_out(w, idx, out, lse, list(range(w.n_q)), TOL[dtype])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [dict(hq=16, dqk=64, dv=64, hi=4, di=32, topk=37,
                                        lengths=(300, 212)),
                                   dict(hq=64, dqk=576, dv=512, hi=8, di=128, topk=100,
                                        lengths=(700,))])
def test_tiny_token_indexer_and_attention(shape, dtype):
    w = tiny_token_workload(seed=7, dtype=dtype, **shape)
    _say("tiny token", shape, dtype)
    d = upload(w)
    idx, score = csa.dsa_indexer_topk(d["iq"], d["ik"], d["w"], d["layout"], w.topk,
                                      return_score=True)
    torch.cuda.synchronize()
    idx_np = idx.cpu().numpy()
    rows = list(range(w.n_q))
    check_token_indices(w, rows, idx_np)
    out, lse = _attn(w, d, idx, out_dtype=torch.float32)
    _check_out(w, idx_np[:, None, :], out, lse, rows, TOL[dtype])


def test_token_mode_per_head_index_and_pads():
    w = tiny_token_workload(seed=8, hq=8, dqk=64, dv=64, lengths=(256,), dtype="bf16")
    _say("token per-head idx")
    rng = np.random.default_rng(8)
    idx = rng.integers(-5, w.n_kv + 5, size=(w.n_q, w.hq, 70)).astype(np.int32)
    d = upload(w)
    out, lse = _attn(w, d, torch.from_numpy(idx).cuda(), out_dtype=torch.float32)
    _check_out(w, idx, out, lse, list(range(w.n_q)), TOL["bf16"])


def test_summary_merge_matches_oracle():
    _say("summary_merge")
    rng = np.random.default_rng(9)
    P, R, dv = 5, 300, 40
    m = (rng.standard_normal((P, R)) * 4).astype(np.float32)
    m[rng.random((P, R)) < 0.3] = -np.inf  # neutral parts
    m[:, :7] = -np.inf                     # rows with no contribution at all
    m[:, 7:20] += 500.0                    # large maxima: unshifted exp would overflow
    l = np.where(np.isinf(m), 0.0, rng.random((P, R)) * 3 + 1).astype(np.float32)
    z = np.where(np.isinf(m)[..., None], 0.0,
                 rng.standard_normal((P, R, dv))).astype(np.float32)
    res = csa.summary_merge(torch.from_numpy(m).cuda(), torch.from_numpy(l).cuda(),
                            torch.from_numpy(z).cuda(), finalize=True, merged=True)
    torch.cuda.synchronize()
    mo, lo, zo = oracle.merge_parts(m, l, z)
    got_m = res["m"].cpu().numpy()
    assert np.array_equal(np.isinf(got_m), np.isinf(mo))
    fin = np.isfinite(mo)
    np.testing.assert_allclose(got_m[fin], mo[fin], rtol=1e-6)
    np.testing.assert_allclose(res["l"].cpu().numpy(), lo, rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(res["z"].cpu().numpy(), zo, rtol=1e-5, atol=1e-5)
    o = res["o"].cpu().numpy()
    lse = res["lse"].cpu().numpy()
    assert not np.isnan(o).any() and not np.isnan(lse).any()
    for r in range(R):
        o_ref, lse_ref = oracle.finalize((mo[r], lo[r], zo[r]))
        np.testing.assert_allclose(o[r], o_ref, rtol=1e-5, atol=1e-5)
        if np.isfinite(lse_ref):
            assert abs(lse[r] - lse_ref) < 1e-4
        else:
            assert lse[r] == -np.inf and not o[r].any()


def test_rows_without_keys_and_all_masked_rows():
    w = tiny_block_workload(seed=10, layout="all", lengths=(256, 256), hq=4, hkv=2, d=64,
                            block=64, topk=2, dtype="bf16")
    _say("no-key rows")
    q_seq = w.q_seq.copy()
    q_pos = w.q_pos.copy()
    q_seq[5] = 1        # sequence 1 starts after position 5
    q_seq[200] = 9      # no such sequence
    q_pos[201] = 9999   # beyond the stream
    w.q_seq, w.q_pos = q_seq, q_pos
    d = upload(w)
    idx = csa.moba_gate_topk(d["q"], d["k"], d["layout"], w.block_size, w.topk)
    torch.cuda.synchronize()
    idx_np = idx.cpu().numpy()
    for r in (5, 200, 201):
        assert (idx_np[r] == -1).all()
    check_moba_indices(w, idx_np)
    out, lse = _attn(w, d, idx, out_dtype=torch.float32)
    for r in (5, 200, 201):
        assert not out[r].any() and (lse[r] == -np.inf).all()
    _check_out(w, idx_np, out, lse, list(range(w.n_q)), TOL["bf16"])
    # index rows holding only pads and future blocks: no key, no NaN
    idx2 = np.full_like(idx_np, -1)
    idx2[:, :, 0] = w.n_kv - w.block_size
    out2, lse2 = _attn(w, d, torch.from_numpy(idx2).cuda(), out_dtype=torch.float32)
    assert not np.isnan(out2).any() and not np.isnan(lse2).any()
    _check_out(w, idx2, out2, lse2, list(range(w.n_q)), TOL["bf16"])


def test_ties_all_zero_keys_pick_lowest():
    w = tiny_block_workload(seed=11, layout="all", lengths=(256,), hq=4, hkv=2, d=64,
                            block=32, topk=3, dtype="bf16")
    w.k = np.zeros_like(w.k)
    _say("ties")
    d = upload(w)
    idx = csa.moba_gate_topk(d["q"], d["k"], d["layout"], w.block_size, w.topk).cpu().numpy()
    for i in range(w.n_q):
        own = (int(w.q_pos[i]) // 32) * 32
        expect = list(range(0, min(own, 96), 32)) + [own]
        for h in range(w.hq):
            assert [x for x in idx[i, h] if x >= 0] == expect
    wt = tiny_token_workload(seed=12, lengths=(200,), topk=17, dtype="bf16")
    wt.iq = -np.ones_like(wt.iq)
    wt.ik = np.ones_like(wt.ik)
    dt = upload(wt)
    idx = csa.dsa_indexer_topk(dt["iq"], dt["ik"], dt["w"], dt["layout"], wt.topk).cpu().numpy()
    for i in range(wt.n_q):
        n = int(wt.q_pos[i]) + 1
        assert [x for x in idx[i] if x >= 0] == list(range(min(n, wt.topk)))


# Crafted indexer inputs whose logits are exact: head 0 has weight 1 and query
# e_0, every other head weight 0 and query 0, and key j is (v_j, 0, ..., 0) with
# v_j >= 0 a bf16 value, so logit(i, j) = v_j in any precision.  The selection
# is then unique (ties to the lower index) and must match the oracle bit for bit.
SELECT_CASES = {
    # many equal bf16 values around the k-th: resolved by the per-bin ranking
    "bf16_ties": dict(lengths=(6000,), topk=1000, values="bf16"),
    # four distinct values, thousands of ties in the threshold bin: radix resolution
    "four_values": dict(lengths=(5000,), topk=700, values="four"),
    # a constant row: everything ties, the lowest indices win
    "constant": dict(lengths=(3000,), topk=300, values="constant"),
    # rows longer than the register-resident capacity take the long-row kernel
    "long_rows": dict(lengths=(18000,), topk=2048, values="bf16"),
}


@pytest.mark.parametrize("case", list(SELECT_CASES))
def test_token_select_crafted_logits(case):
    c = SELECT_CASES[case]
    n_kv = sum(c["lengths"])
    rng = np.random.default_rng(31)
    pos = np.unique(np.concatenate([rng.integers(0, n_kv, 40), [0, 1, c["topk"] - 1,
                                    c["topk"], c["topk"] + 1, n_kv - 1]])).astype(np.int32)
    w = tiny_token_workload(seed=31, lengths=c["lengths"], positions=pos, hq=4, dqk=64, dv=64,
                            hi=32, di=64, topk=c["topk"], dtype="bf16")
    if c["values"] == "bf16":
        v = torch.from_numpy(rng.uniform(0, 100, n_kv).astype(np.float32)).bfloat16().float()
        v = v.numpy()
    elif c["values"] == "four":
        v = rng.integers(0, 4, n_kv).astype(np.float32)
    else:
        v = np.full(n_kv, 5.0, np.float32)
    w.iq = np.zeros_like(w.iq)
    w.iq[:, 0, 0] = 1.0
    w.ik = np.zeros_like(w.ik)
    w.ik[:, 0] = v
    w.w = np.zeros_like(w.w)
    w.w[:, 0] = 1.0
    _say("crafted select", case, "n_kv", n_kv, "rows", len(pos), "topk", w.topk)
    d = upload(w)
    idx, score = csa.dsa_indexer_topk(d["iq"], d["ik"], d["w"], d["layout"], w.topk,
                                      return_score=True)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    score = score.cpu().numpy()
    ref, _, _ = oracle.indexer_topk(w.iq, w.ik, w.w, w.q_pos, w.q_seq, w.cu_seqlens, w.topk)
    bad = [i for i in range(len(pos)) if not np.array_equal(idx[i], ref[i])]
    assert not bad, f"rows {bad[:5]} differ, e.g. row {bad[0]} at pos {pos[bad[0]]}"
    sel = idx >= 0
    assert np.array_equal(score[sel], v[idx[sel]])
    assert np.isneginf(score[~sel]).all()


def test_determinism_bitwise():
    w = tiny_block_workload(seed=13, layout="all", lengths=(1000, 537), hq=8, hkv=2, d=128,
                            block=64, topk=3, dtype="bf16")
    _say("determinism")
    d = upload(w)
    outs = []
    for _ in range(2):
        idx = csa.moba_gate_topk(d["q"], d["k"], d["layout"], w.block_size, w.topk)
        out, lse = csa.sparse_attn_fwd_shard(d["q"], d["k"], d["v"], d["layout"],
                                             csa.CSA_SEL_BLOCK, idx, block_size=w.block_size,
                                             softmax_scale=w.scale)
        torch.cuda.synchronize()
        outs.append((idx.cpu(), out.cpu(), lse.cpu()))
    for a, b in zip(*outs):
        assert torch.equal(a, b)


@pytest.mark.parametrize("mode", ["block", "token"])
def test_graph_capture_replays_match_eager(mode):
    """A whole step (selection + attention) captured as a HIP graph reproduces the
    eager result bit for bit on every replay, with eager work and synchronizations
    between the replays."""
    if mode == "block":
        w = tiny_block_workload(seed=21, layout="all", lengths=(1000, 537), hq=8, hkv=2,
                                d=128, block=64, topk=3, dtype="bf16")
    else:
        w = tiny_token_workload(seed=22, lengths=(700, 300), hq=64, dqk=128, dv=128, hi=8,
                                di=64, topk=97, dtype="bf16")
    _say("graph capture", mode)
    d = upload(w)
    sel_mode = csa.CSA_SEL_BLOCK if mode == "block" else csa.CSA_SEL_TOKEN

    def step():
        if mode == "block":
            idx = csa.moba_gate_topk(d["q"], d["k"], d["layout"], w.block_size, w.topk)
        else:
            idx = csa.dsa_indexer_topk(d["iq"], d["ik"], d["w"], d["layout"], w.topk)
        out, lse = csa.sparse_attn_fwd_shard(d["q"], d["k"], d["v"], d["layout"], sel_mode, idx,
                                             block_size=w.block_size, softmax_scale=w.scale)
        return idx, out, lse

    ref = [t.clone() for t in step()]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        got = step()
    torch.cuda.synchronize()
    for _ in range(4):
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, got):
            assert torch.equal(a, b)
        step()  # eager work between replays
        torch.cuda.synchronize()


# --------------------------------------------------------------------------------
# the five named workloads at full size
# --------------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["dense_f32", "moba_mha_8k", "moba_gqa_zigzag_32k",
                                  "moba_thd_64k"])
def test_named_block_workload(name):
    w = make_workload(name)
    _say("workload", name, w.q.shape, w.k.shape)
    d = upload(w)
    idx = csa.moba_gate_topk(d["q"], d["k"], d["layout"], w.block_size, w.topk)
    torch.cuda.synchronize()
    idx_np = idx.cpu().numpy()
    counts = check_moba_indices(w, idx_np)
    _say(name, "index categories", counts)
    # rows: sequence starts (own block only, partially masked), shard edges, random
    cu = w.cu_seqlens
    starts = [i for i in range(w.n_q) if int(w.q_pos[i]) in set(cu[:-1].tolist())]
    rows = sample_rows(w.n_q, 48, seed=1, must=[0, w.n_q - 1, w.n_q // 2, *starts[:8]])
    out, lse = _attn(w, d, idx, out_dtype=torch.float32)
    err = _check_out(w, idx_np, out, lse, rows, TOL[w.dtype])
    _say(name, "fp32-out max abs err", err)
    if w.dtype == "bf16":
        out_b, lse_b = _attn(w, d, idx, out_dtype=torch.bfloat16)
        err_b = _check_out(w, idx_np, out_b, lse_b, rows, TOL["bf16"])
        _say(name, "bf16-out max abs err", err_b)


def test_named_dsa_workload():
    w = make_workload("dsa_mla_16k")
    _say("workload dsa_mla_16k")
    d = upload(w)
    assert d["v"].data_ptr() == d["k"].data_ptr()  # aliased latent value
    idx = csa.dsa_indexer_topk(d["iq"], d["ik"], d["w"], d["layout"], w.topk)
    torch.cuda.synchronize()
    idx_np = idx.cpu().numpy()
    rows = sample_rows(w.n_q, 12, seed=2, must=[0, w.n_q - 1])
    counts = check_token_indices(w, rows, idx_np[rows])
    _say("dsa index categories", counts)
    out, lse = _attn(w, d, idx, out_dtype=torch.bfloat16)
    err = _check_out(w, idx_np[:, None, :], out, lse, rows, TOL["bf16"])
    _say("dsa bf16-out max abs err", err)

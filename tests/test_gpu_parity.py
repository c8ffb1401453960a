"""GPU parity: every C-ABI entry point against the fp64 oracle (MI355X only).

Inputs are the seeded workloads of ``csa_inputs``; the oracle reads the same
values.  Index outputs follow the margin criterion and outputs the tolerances
of tests/parity.py.  Every output tensor is pre-filled with NaN (index
outputs with a sentinel) so that an element the GPU never writes fails.  Small
cases and the five named workloads at full size (in the launch configuration
the benchmark uses) check every row: every selection against the margin
criterion, every selected score against the oracle's, and every (row, head)
output and log-sum-exp against the oracle evaluated on the GPU's selection
(the full-size oracle runs in worker processes, tests/oracle_pool.py).
"""

import numpy as np
import pytest
import torch

import oracle
from csa_inputs import (make_workload, tiny_block_workload, tiny_token_workload,
                        contiguous_positions, zigzag_positions)
from parity import (TOL, upload, check_moba_indices, check_moba_scores, check_token_indices,
                    poisoned, INDEXER_SCORE_REL)
from oracle_pool import OraclePool, run_local, _dsa_check

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

if torch.cuda.is_available():
    import context_sparse_attention_amd as csa


def _say(*a):
    print("[case]", *a, flush=True)


def _attn(w, d, idx, out_dtype=None, mode=None):
    """Attention into NaN-filled out / lse tensors; (out as float32 numpy, lse)."""
    mode = (csa.CSA_SEL_BLOCK if w.mode == "block" else csa.CSA_SEL_TOKEN) if mode is None else mode
    out_dtype = out_dtype or d["q"].dtype
    out = poisoned((w.n_q, w.hq, w.dv), out_dtype)
    lse = poisoned((w.n_q, w.hq), torch.float32)
    csa.sparse_attn_fwd_shard(d["q"], d["k"], d["v"], d["layout"], mode, idx,
                              block_size=w.block_size, softmax_scale=w.scale, out=out, lse=lse)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


def _gate(w, d):
    """Gate into sentinel / NaN-filled idx and score tensors (numpy results)."""
    shape = (w.n_q, w.hq, w.topk + 1)
    idx, score = csa.moba_gate_topk(d["q"], d["k"], d["layout"], w.block_size, w.topk,
                                    idx=poisoned(shape, torch.int32),
                                    score=poisoned(shape, torch.float32))
    torch.cuda.synchronize()
    return idx, idx.cpu().numpy(), score.cpu().numpy()


def _indexer(w, d):
    shape = (w.n_q, w.topk)
    idx, score = csa.dsa_indexer_topk(d["iq"], d["ik"], d["w"], d["layout"], w.topk,
                                      idx=poisoned(shape, torch.int32),
                                      score=poisoned(shape, torch.float32))
    torch.cuda.synchronize()
    return idx, idx.cpu().numpy(), score.cpu().numpy()


def _dsa_arrays(w, idx_np, score_np):
    return dict(iq=w.iq, ik=w.ik, w=w.w, q_pos=w.q_pos, q_seq=w.q_seq, cu=w.cu_seqlens,
                idx=idx_np, score=score_np)


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
    idx, idx_np, score_np = _gate(w, d)
    gate = oracle.gate_scores(w.q, w.k, w.q_pos, w.q_seq, w.cu_seqlens, w.block_size)
    counts = check_moba_indices(w, idx_np, gate)
    assert counts["exact"] > 0
    check_moba_scores(w, gate, idx_np, score_np)
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


TINY_TOKEN = [
    # general-shape kernel (16 heads)
    dict(hq=16, dqk=64, dv=64, hi=4, di=32, topk=37, lengths=(300, 212)),
    # MFMA kernel, one wave per workgroup (32 heads)
    dict(hq=32, dqk=128, dv=128, hi=4, di=64, topk=50, lengths=(400,)),
    # absorbed-MLA widths, 16 heads a wave: two waves (32 heads)
    dict(hq=32, dqk=576, dv=512, hi=8, di=128, topk=60, lengths=(300,)),
    # absorbed-MLA widths, four waves (64 heads)
    dict(hq=64, dqk=576, dv=512, hi=8, di=128, topk=100, lengths=(700,)),
    # absorbed-MLA widths, eight waves (128 heads)
    dict(hq=128, dqk=576, dv=512, hi=8, di=128, topk=70, lengths=(200, 150)),
]


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", range(len(TINY_TOKEN)))
def test_tiny_token_indexer_and_attention(shape, dtype, out):
    w = tiny_token_workload(seed=7, dtype=dtype, **TINY_TOKEN[shape])
    _say("tiny token", TINY_TOKEN[shape], dtype, "out", out)
    d = upload(w)
    idx, idx_np, score_np = _indexer(w, d)
    rows = list(range(w.n_q))
    res = run_local(_dsa_arrays(w, idx_np, score_np), _dsa_check, rows,
                    dict(topk=w.topk, score_rel=INDEXER_SCORE_REL))
    assert res["n_fail"] == 0, res["fails"]
    assert res["counts"]["exact"] > 0
    out_dtype = torch.float32 if out == "f32" else torch.bfloat16
    tol = TOL[dtype] if out == "f32" else TOL["bf16"]
    got, lse = _attn(w, d, idx, out_dtype=out_dtype)
    _check_out(w, idx_np[:, None, :], got, lse, rows, tol)


def test_token_mode_per_head_index_and_pads():
    w = tiny_token_workload(seed=8, hq=8, dqk=64, dv=64, lengths=(256,), dtype="bf16")
    _say("token per-head idx")
    rng = np.random.default_rng(8)
    idx = rng.integers(-5, w.n_kv + 5, size=(w.n_q, w.hq, 70)).astype(np.int32)
    d = upload(w)
    out, lse = _attn(w, d, torch.from_numpy(idx).cuda(), out_dtype=torch.float32)
    _check_out(w, idx, out, lse, list(range(w.n_q)), TOL["bf16"])


def _mla_slots(rng, pos, n_kv, width, hot, hot_slot):
    """Caller-made token selections: permitted keys, pads, future (masked) keys and
    repeats of the previous slot; the hot key at hot_slot where the row may see it;
    one row of pads only and one of future keys only."""
    n_q = len(pos)
    idx = np.full((n_q, width), -1, np.int32)
    for i in range(n_q):
        p = int(pos[i])
        for s in range(width):
            u = rng.random()
            if u < 0.1:
                continue
            if u < 0.2 and p + 1 < n_kv:
                idx[i, s] = rng.integers(p + 1, n_kv)
            elif u < 0.3 and s > 0:
                idx[i, s] = idx[i, s - 1]
            else:
                idx[i, s] = rng.integers(0, p + 1)
        if p >= hot and width > hot_slot:
            idx[i, hot_slot] = hot
    idx[3] = -1
    idx[11] = rng.integers(pos[11] + 1, n_kv, size=width)
    return idx


@pytest.mark.parametrize("hq", [64, 128])
def test_token_mla_widths_edge_cases(hq):
    """Absorbed-MLA widths (16 heads a wave; at 128 heads the two waves of a SIMD
    share P and form P V one tile late, one of them starting a few steps of it
    before its scores): caller-made selections of 1, 5, 33 and 97 slots (one to
    four 32-key tiles)
    with pads, repeats, future keys and rows without keys, and a key whose score
    dwarfs the rest in the third tile, so that the running maximum moves after
    the first tile; bf16 and f32 outputs, and the result repeats bit for bit."""
    w = tiny_token_workload(seed=41, lengths=(300,), hq=hq, dqk=576, dv=512, hi=8, di=128,
                            topk=16, dtype="bf16")
    hot = 150
    w.k[hot, :, 512:] *= 32.0  # rope columns only: scores grow, the value row does not
    d = upload(w)
    rng = np.random.default_rng(41)
    for width in (1, 5, 33, 97):
        idx_np = _mla_slots(rng, w.q_pos, w.n_kv, width, hot, hot_slot=70)
        idx = torch.from_numpy(idx_np).cuda()
        _say("token mla edges", hq, "width", width)
        for out_dtype in (torch.float32, torch.bfloat16):
            out, lse = _attn(w, d, idx, out_dtype=out_dtype)
            for r in (3, 11):
                assert not out[r].any() and (lse[r] == -np.inf).all()
            tol = TOL["bf16"]
            _check_out(w, idx_np[:, None, :], out, lse, list(range(w.n_q)), tol)
            again = _attn(w, d, idx, out_dtype=out_dtype)
            assert np.array_equal(out, again[0]) and np.array_equal(lse, again[1])


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
# the five named workloads at full size: every row
# --------------------------------------------------------------------------------

def _attn_arrays(w, idx_np, outs):
    a = dict(q=w.q, k=w.k, v=w.value, q_pos=w.q_pos, q_seq=w.q_seq, cu=w.cu_seqlens,
             idx=idx_np if idx_np.ndim == 3 else idx_np[:, None, :])
    a.update(outs)
    return a


def _pool_attn_check(w, idx_np, outs, targets):
    with OraclePool(_attn_arrays(w, idx_np, outs)) as pool:
        _say(w.name, "oracle workers", pool.processes)
        res = pool.attn_check(range(w.n_q), dict(mode=w.mode, scale=w.scale,
                                                 block_size=w.block_size, targets=targets))
    for (name, _, tol), r in zip(targets, res):
        _say(w.name, name, "rows", w.n_q, "(row, head) pairs", r["pairs"], "without keys",
             r["no_key_pairs"], "max abs err", f"{r['max_err']:.3e}", "max lse err",
             f"{r['max_lse_err']:.3e}", "tol", tol)
        assert not r["fails"], r["fails"][:5]
        assert r["pairs"] == w.n_q * w.hq


@pytest.mark.parametrize("name", ["dense_f32", "moba_mha_8k", "moba_gqa_zigzag_32k",
                                  "moba_thd_64k"])
def test_named_block_workload(name):
    w = make_workload(name)
    _say("workload", name, w.q.shape, w.k.shape)
    d = upload(w)
    family = csa.sparse_attn_fwd_shard_kernel(d["q"], d["k"], d["v"], d["layout"],
                                              csa.CSA_SEL_BLOCK, w.hq, w.topk + 1,
                                              w.block_size, w.scale)
    _say(name, "attention kernel family", family)
    assert family == ("generic" if w.dtype == "f32" else "block_mfma")
    idx, idx_np, score_np = _gate(w, d)
    gate = oracle.gate_scores(w.q, w.k, w.q_pos, w.q_seq, w.cu_seqlens, w.block_size)
    counts = check_moba_indices(w, idx_np, gate)
    _say(name, "index categories over", w.n_q, "rows x", w.hq, "heads:", counts)
    worst, n = check_moba_scores(w, gate, idx_np, score_np)
    _say(name, "gate scores compared", n, "max abs err", f"{worst:.3e}")
    outs, targets = {}, []
    out_f, lse_f = _attn(w, d, idx, out_dtype=torch.float32)
    outs.update(out_f32=out_f, lse_f32=lse_f)
    targets.append(("out_f32", "lse_f32", TOL[w.dtype]))
    if w.dtype == "bf16":
        out_b, lse_b = _attn(w, d, idx, out_dtype=torch.bfloat16)
        outs.update(out_bf16=out_b, lse_bf16=lse_b)
        targets.append(("out_bf16", "lse_bf16", TOL["bf16"]))
    _pool_attn_check(w, idx_np, outs, targets)


def test_named_dsa_workload():
    w = make_workload("dsa_mla_16k")
    _say("workload dsa_mla_16k")
    d = upload(w)
    assert d["v"].data_ptr() == d["k"].data_ptr()  # aliased latent value
    family = csa.sparse_attn_fwd_shard_kernel(d["q"], d["k"], d["v"], d["layout"],
                                              csa.CSA_SEL_TOKEN, 1, w.topk, 0, w.scale)
    _say("dsa attention kernel family", family)
    assert family == "token_mfma"
    idx, idx_np, score_np = _indexer(w, d)
    with OraclePool(_dsa_arrays(w, idx_np, score_np)) as pool:
        res = pool.dsa_check(range(w.n_q), dict(topk=w.topk, score_rel=INDEXER_SCORE_REL))
    _say("dsa indexer over", w.n_q, "rows:", res["counts"], "failures", res["n_fail"],
         "max score err", f"{res['max_score_err']:.3e}")
    assert res["n_fail"] == 0, res["fails"]
    assert sum(res["counts"].values()) == w.n_q
    out_b, lse_b = _attn(w, d, idx, out_dtype=torch.bfloat16)
    _pool_attn_check(w, idx_np, dict(out_bf16=out_b, lse_bf16=lse_b),
                     [("out_bf16", "lse_bf16", TOL["bf16"])])


@pytest.mark.parametrize("layout", ["contiguous", "zigzag"])
def test_shards_stitch_to_the_full_run(layout):
    """Megatron-LM issue #4878, "Strategy: allgather CP mode", planned test: a
    shard at its causal offset equals the matching slice of a full single-rank
    run.  Every rank of a cp=4 split (contiguous or zigzag) is run on its own
    and the shards, stitched back by global position, are compared with the
    cp=1 run of the same stream: selections bit for bit, outputs within the
    bf16 tolerance (and reported when bitwise equal)."""
    cp = 4
    w = tiny_block_workload(seed=41, layout="all", lengths=(4096,), hq=8, hkv=2, d=128,
                            block=256, topk=3, dtype="bf16")
    _say("stitch", layout)
    full = upload(w)
    idx_full, idx_full_np, score_full = _gate(w, full)
    out_full, lse_full = _attn(w, full, idx_full, out_dtype=torch.bfloat16)
    seen = np.zeros(w.n_q, np.int64)
    bitwise = True
    make = contiguous_positions if layout == "contiguous" else zigzag_positions
    for rank in range(cp):
        pos = make(w.n_kv, cp, rank)
        seen[pos] += 1
        sw = tiny_block_workload(seed=41, layout="all", lengths=(4096,), hq=8, hkv=2, d=128,
                                 block=256, topk=3, dtype="bf16")
        sw.q, sw.q_pos, sw.q_seq = w.q[pos], pos.astype(np.int32), w.q_seq[pos]
        sd = upload(sw)
        idx_s, idx_s_np, score_s = _gate(sw, sd)
        assert np.array_equal(idx_s_np, idx_full_np[pos]), f"rank {rank}: selections differ"
        assert np.array_equal(score_s, score_full[pos]), f"rank {rank}: gate scores differ"
        out_s, lse_s = _attn(sw, sd, idx_s, out_dtype=torch.bfloat16)
        assert np.isfinite(out_s).all() and not np.isnan(lse_s).any()
        err = np.abs(out_s - out_full[pos]).max()
        assert err <= TOL["bf16"], f"rank {rank}: max abs err {err:.3e}"
        np.testing.assert_allclose(lse_s, lse_full[pos], rtol=0, atol=1e-4)
        bitwise &= bool(np.array_equal(out_s, out_full[pos]) and
                        np.array_equal(lse_s, lse_full[pos]))
    assert (seen == 1).all()
    _say("stitch", layout, "shards equal the full run bit for bit:", bitwise)

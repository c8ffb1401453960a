"""CPU checks of the full-size parity machinery (tests/oracle_pool.py).

The GPU tests hand the GPU's results to worker processes that compare them
with the oracle.  Here the "GPU results" are the oracle's own (rounded to
float32 as the GPU's would be), so every check must pass; a planted error in
one output element, one index and one score must each be reported.
"""

import numpy as np

import oracle
from csa_inputs import tiny_block_workload, tiny_token_workload
from oracle_pool import OraclePool, run_local, _attn_check, _dsa_check


def _block_case():
    w = tiny_block_workload(seed=3, layout="all", lengths=(70, 90), hq=4, hkv=2, d=16,
                            block=16, topk=2)
    gate = oracle.gate_scores(w.q, w.k, w.q_pos, w.q_seq, w.cu_seqlens, w.block_size)
    idx = oracle.select_blocks(gate, w.topk)
    out, lse = oracle.shard_forward(w.q, w.k, w.value, w.q_pos, w.q_seq, w.cu_seqlens,
                                    "block", idx, w.scale, w.block_size)
    arrays = dict(q=w.q, k=w.k, v=w.value, q_pos=w.q_pos, q_seq=w.q_seq, cu=w.cu_seqlens,
                  idx=idx, out=out.astype(np.float32), lse=lse.astype(np.float32))
    params = dict(mode="block", scale=w.scale, block_size=w.block_size,
                  targets=[("out", "lse", 1e-5)])
    return w, arrays, params


def test_pool_attention_check_passes_on_oracle_results_and_catches_a_planted_error():
    w, arrays, params = _block_case()
    with OraclePool(arrays, processes=2) as pool:
        (res,) = pool.attn_check(range(w.n_q), params)
    assert not res["fails"] and res["pairs"] == w.n_q * w.hq
    assert res["max_err"] < 1e-6
    (local,) = run_local(arrays, _attn_check, range(w.n_q), params)
    assert local["max_err"] == res["max_err"]
    bad = dict(arrays)
    bad["out"] = arrays["out"].copy()
    bad["out"][17, 2, 5] += 1e-3
    (res,) = run_local(bad, _attn_check, range(w.n_q), params)
    assert any("row 17 head 2 col 5" in f for f in res["fails"])
    bad["out"] = arrays["out"].copy()
    bad["out"][40, 1, 0] = np.nan  # an element the GPU would not have written
    (res,) = run_local(bad, _attn_check, range(w.n_q), params)
    assert any("non-finite" in f for f in res["fails"])


def _token_case():
    w = tiny_token_workload(seed=5, lengths=(60, 40), hi=3, di=8, topk=9)
    idx, logits, los = oracle.indexer_topk(w.iq, w.ik, w.w, w.q_pos, w.q_seq, w.cu_seqlens,
                                           w.topk)
    score = np.full(idx.shape, -np.inf, np.float32)
    for r in range(w.n_q):
        sel = idx[r] >= 0
        score[r, sel] = logits[r][idx[r, sel] - los[r]]
    arrays = dict(iq=w.iq, ik=w.ik, w=w.w, q_pos=w.q_pos, q_seq=w.q_seq, cu=w.cu_seqlens,
                  idx=idx, score=score)
    return w, arrays, dict(topk=w.topk, score_rel=5e-5)


def test_dsa_check_passes_on_oracle_results_and_catches_planted_errors():
    w, arrays, params = _token_case()
    with OraclePool(arrays, processes=2) as pool:
        res = pool.dsa_check(range(w.n_q), params)
    assert res["n_fail"] == 0, res["fails"]
    assert res["counts"]["exact"] == w.n_q
    # a selection swapped for a clearly worse key
    bad = dict(arrays, idx=arrays["idx"].copy())
    r = 80
    lo = int(w.cu_seqlens[w.q_seq[r]])
    L = oracle.indexer_logits_row(w.iq[r], w.ik, w.w[r], lo, int(w.q_pos[r]))
    worst = lo + int(np.argmin(L))
    row = [x for x in bad["idx"][r] if x >= 0][1:] + [worst]
    bad["idx"][r, :len(row)] = np.sort(row)
    res = run_local(bad, _dsa_check, range(w.n_q), params)
    assert res["n_fail"] == 1 and "row 80" in res["fails"][0]
    # a selected logit off by more than the rounding bound
    bad = dict(arrays, score=arrays["score"].copy())
    bad["score"][30, 2] *= 1.001
    res = run_local(bad, _dsa_check, range(w.n_q), params)
    assert res["n_fail"] == 1 and "score error" in res["fails"][0]

"""GPU parity of sparse_attn_bwd_shard against the fp64 oracle (MI355X only).

The forward runs first (its output and log-sum-exp feed the backward, as in
training); dO is seeded N(0, 1).  Every dq, dk and dv element is compared with
``oracle.shard_backward`` on the same selection: max-abs error within 1e-5 for
fp32 inputs and 2e-2 for bf16 inputs, times max(1, the largest |element| of the
oracle's tensor) - a gradient element sums many (row, head) terms, so its fp32
rounding scales with the gradient's size.  Outputs are pre-filled with NaN so that an element the
GPU never writes fails.  At full size (every bf16 workload) the oracle's dq of
sampled rows is compared; in block mode also dk and dv of whole sampled key
blocks (the oracle on every row that selects the block); for the fp32-operand
kernels two identities hold at any size: for each key head, the dk rows sum to
zero (the softmax Jacobian's rows sum to zero) and the dv rows sum to the dO
rows of the (row, head) pairs that have keys (each such softmax sums to one).
"""

import numpy as np
import pytest
import torch

import oracle
from csa_inputs import make_workload, tiny_block_workload, tiny_token_workload
from parity import TOL, upload, poisoned
from oracle_pool import OraclePool

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

if torch.cuda.is_available():
    import context_sparse_attention_amd as csa


def _say(*a):
    print("[case]", *a, flush=True)


def _family(w, d, idx):
    mode = csa.CSA_SEL_BLOCK if w.mode == "block" else csa.CSA_SEL_TOKEN
    heads = 1 if idx.dim() == 2 else idx.shape[1]
    return csa.sparse_attn_bwd_shard_kernel(d["q"], d["k"], d["v"], d["layout"], mode, heads,
                                            idx.shape[-1], w.block_size)


def _fwd_bwd(w, d, idx, dout_np, out_dtype=torch.float32):
    mode = csa.CSA_SEL_BLOCK if w.mode == "block" else csa.CSA_SEL_TOKEN
    out, lse = csa.sparse_attn_fwd_shard(d["q"], d["k"], d["v"], d["layout"], mode, idx,
                                         block_size=w.block_size, softmax_scale=w.scale,
                                         out_dtype=out_dtype)
    dout = torch.from_numpy(dout_np.astype(np.float32)).cuda().to(out_dtype)
    dq = poisoned((w.n_q, w.hq, w.dqk), torch.float32)
    dk = poisoned((w.n_kv, w.hkv, w.dqk), torch.float32)
    dv = poisoned((w.n_kv, w.hkv, w.dv), torch.float32)
    csa.sparse_attn_bwd_shard(d["q"], d["k"], d["v"], d["layout"], mode, idx, out, dout, lse,
                              block_size=w.block_size, softmax_scale=w.scale, dq=dq, dk=dk,
                              dv=dv)
    torch.cuda.synchronize()
    return dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy(), dout.float().cpu().numpy()


def _compare(w, idx_np, dout, got, tol, label):
    dq, dk, dv = got
    for name, a in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert np.isfinite(a).all(), f"{label}: {name} has unwritten or non-finite elements"
    ref = oracle.shard_backward(w.q, w.k, w.value, w.q_pos, w.q_seq, w.cu_seqlens, w.mode,
                                idx_np, w.scale, dout, w.block_size)
    errs = {}
    for name, a, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        # a gradient element sums many (row, head) terms: its fp32 rounding grows
        # with the tensor's scale, so the bar is relative to its largest element
        scale = max(1.0, float(np.abs(r).max()))
        errs[name] = (float(np.abs(a - r).max()), scale)
        assert errs[name][0] <= tol * scale, \
            f"{label}: {name} max abs err {errs[name][0]:.3e} > {tol} x {scale:.3g}"
    _say(label, {k: f"{v[0]:.2e} (scale {v[1]:.3g})" for k, v in errs.items()})


BLOCK_CASES = [
    dict(seed=60, lengths=(300, 212), layout="all", hq=4, hkv=2, d=64, block=64, topk=2),
    dict(seed=61, lengths=(512,), layout="zigzag", cp=4, rank=1, hq=8, hkv=2, d=128, block=64,
         topk=3),
    dict(seed=62, lengths=(77, 300, 19, 116), layout="all", hq=4, hkv=4, d=128, block=64,
         topk=4),
    dict(seed=63, lengths=(300, 212), layout="all", hq=4, hkv=2, d=64, block=48, topk=3),
    # lists of several 128-entry chunks, blocks of four 64-key subtiles, ragged ends
    dict(seed=69, lengths=(2500, 1100), layout="zigzag", cp=2, rank=0, hq=8, hkv=2, d=128,
         block=256, topk=3),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", range(len(BLOCK_CASES)))
def test_block_backward_matches_oracle(case, dtype):
    w = tiny_block_workload(dtype=dtype, **BLOCK_CASES[case])
    _say("block backward", case, dtype, w.q.shape, w.k.shape)
    d = upload(w)
    idx = csa.moba_gate_topk(d["q"], d["k"], d["layout"], w.block_size, w.topk)
    idx_np = idx.cpu().numpy()
    # bf16 with D in {64, 128} and per-head index rows: the matrix-core kernels
    assert _family(w, d, idx) == ("block_mfma" if dtype == "bf16" else "generic")
    dout = np.random.default_rng(case).standard_normal((w.n_q, w.hq, w.dv))
    got = _fwd_bwd(w, d, idx, dout)
    _compare(w, idx_np, got[3], got[:3], TOL[dtype], f"block {case} {dtype}")


def test_block_backward_caller_slots_and_bf16_output():
    """Pads, misaligned, future and repeated slots; rows without keys; the forward's
    output in bf16 (D then uses the rounded output: the bf16 tolerance)."""
    w = tiny_block_workload(seed=64, layout="all", lengths=(300, 420, 180), hq=4, hkv=2, d=64,
                            block=64, topk=2, dtype="bf16")
    q_seq = w.q_seq.copy()
    q_seq[7] = 9
    w.q_seq = q_seq
    rng = np.random.default_rng(64)
    W = 6
    idx_np = rng.integers(-3, w.n_kv + 3, size=(w.n_q, w.hq, W)).astype(np.int32)
    for i in range(w.n_q):
        lo = int(w.cu_seqlens[w.q_seq[i]]) if 0 <= w.q_seq[i] < 3 else 0
        for s in range(0, W, 2):
            idx_np[i, :, s] = lo + w.block_size * rng.integers(0, 5, size=w.hq)
    idx_np[::3, :, 1] = idx_np[::3, :, 0]
    _say("block backward caller slots")
    d = upload(w)
    idx = torch.from_numpy(idx_np).cuda()
    assert _family(w, d, idx) == "block_mfma"
    dout = rng.standard_normal((w.n_q, w.hq, w.dv))
    got = _fwd_bwd(w, d, idx, dout, out_dtype=torch.bfloat16)
    assert not got[0][7].any()
    _compare(w, idx_np, got[3], got[:3], TOL["bf16"], "caller slots")


TOKEN_CASES = [
    dict(hq=16, dqk=64, dv=64, hi=4, di=32, topk=37, lengths=(300, 212)),
    dict(hq=64, dqk=576, dv=512, hi=8, di=128, topk=100, lengths=(700,)),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", range(len(TOKEN_CASES)))
def test_token_backward_matches_oracle(case, dtype):
    """Indexer selection shared by all heads; the value aliases the key's first
    columns (absorbed MLA), with dk and dv returned separately."""
    w = tiny_token_workload(seed=65 + case, dtype=dtype, **TOKEN_CASES[case])
    _say("token backward", case, dtype)
    d = upload(w)
    idx = csa.dsa_indexer_topk(d["iq"], d["ik"], d["w"], d["layout"], w.topk)
    # bf16 absorbed-MLA shape (576 / 512): dK and dV on the matrix cores
    mla = dtype == "bf16" and (w.dqk, w.dv) == (576, 512)
    assert _family(w, d, idx) == ("token_mfma" if mla else "generic")
    idx_np = idx.cpu().numpy()[:, None, :]
    dout = np.random.default_rng(case).standard_normal((w.n_q, w.hq, w.dv))
    got = _fwd_bwd(w, d, idx, dout)
    _compare(w, idx_np, got[3], got[:3], TOL[dtype], f"token {case} {dtype}")


def test_token_backward_separate_value_rows_match_aliased():
    """Absorbed-MLA shape with V passed as its own tensor (a copy of the key's first
    512 columns): the separate-value kernel must give the aliased kernel's gradients
    bit for bit, and both the oracle's."""
    w = tiny_token_workload(seed=66, dtype="bf16", **TOKEN_CASES[1])
    _say("token backward separate v")
    d = upload(w)
    idx = csa.dsa_indexer_topk(d["iq"], d["ik"], d["w"], d["layout"], w.topk)
    assert _family(w, d, idx) == "token_mfma"
    mode = csa.CSA_SEL_TOKEN
    out, lse = csa.sparse_attn_fwd_shard(d["q"], d["k"], d["v"], d["layout"], mode, idx,
                                         softmax_scale=w.scale)
    dout_np = np.random.default_rng(5).standard_normal((w.n_q, w.hq, w.dv))
    dout = torch.from_numpy(dout_np.astype(np.float32)).cuda()
    got = []
    for v in (d["v"], d["v"].contiguous()):
        dq = poisoned((w.n_q, w.hq, w.dqk), torch.float32)
        dk = poisoned((w.n_kv, w.hkv, w.dqk), torch.float32)
        dv = poisoned((w.n_kv, w.hkv, w.dv), torch.float32)
        csa.sparse_attn_bwd_shard(d["q"], d["k"], v, d["layout"], mode, idx, out, dout, lse,
                                  softmax_scale=w.scale, dq=dq, dk=dk, dv=dv)
        torch.cuda.synchronize()
        got.append((dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()))
    assert d["v"].data_ptr() == d["k"].data_ptr()
    for name, a, b in zip(("dq", "dk", "dv"), got[0], got[1]):
        assert np.array_equal(a, b), f"{name}: separate-value kernel differs from aliased"
    _compare(w, idx.cpu().numpy()[:, None, :], dout_np.astype(np.float32), got[1], TOL["bf16"],
             "token separate v")


def test_token_backward_per_head_index_with_pads_and_repeats():
    w = tiny_token_workload(seed=67, hq=8, dqk=64, dv=64, lengths=(256,), dtype="bf16")
    rng = np.random.default_rng(67)
    idx_np = rng.integers(-5, w.n_kv + 5, size=(w.n_q, w.hq, 70)).astype(np.int32)
    idx_np[:, :, 5] = idx_np[:, :, 4]
    _say("token backward per-head idx")
    d = upload(w)
    dout = rng.standard_normal((w.n_q, w.hq, w.dv))
    got = _fwd_bwd(w, d, torch.from_numpy(idx_np).cuda(), dout)
    _compare(w, idx_np, got[3], got[:3], TOL["bf16"], "token per-head")


@pytest.mark.parametrize("per_head", [False, True])
def test_token_backward_wide_rows(per_head):
    """Index rows of 256 slots or more build the key lists with their counts and
    cursors in LDS (one workgroup per range of rows): the absorbed-MLA shape on the
    matrix cores with a shared index row, and per-head rows with pads, future keys
    and repeated slots on the general kernels; gradients against the oracle, and a
    second call repeats them bit for bit."""
    if per_head:
        w = tiny_token_workload(seed=69, hq=8, dqk=64, dv=64, lengths=(600,), dtype="bf16")
        rng = np.random.default_rng(69)
        idx_np = rng.integers(-5, w.n_kv + 5, size=(w.n_q, w.hq, 300)).astype(np.int32)
        idx_np[:, :, 7] = idx_np[:, :, 3]
        idx = torch.from_numpy(idx_np).cuda()
        family = "generic"
    else:
        w = tiny_token_workload(seed=70, hq=32, dqk=576, dv=512, hi=8, di=128, topk=280,
                                lengths=(400,), dtype="bf16")
        rng = np.random.default_rng(70)
        d0 = upload(w)
        idx = csa.dsa_indexer_topk(d0["iq"], d0["ik"], d0["w"], d0["layout"], w.topk)
        idx_np = idx.cpu().numpy()[:, None, :]
        family = "token_mfma"
    _say("token backward wide rows", "per-head" if per_head else "shared")
    d = upload(w)
    assert _family(w, d, idx) == family
    dout = rng.standard_normal((w.n_q, w.hq, w.dv))
    got = _fwd_bwd(w, d, idx, dout)
    again = _fwd_bwd(w, d, idx, dout)
    for name, a, b in zip(("dq", "dk", "dv"), got[:3], again[:3]):
        assert np.array_equal(a, b), f"{name} differs between two calls"
    _compare(w, idx_np, got[3], got[:3], TOL["bf16"], "token wide rows")


def test_token_backward_many_keys_global_lists():
    """More keys than one workgroup's LDS holds counts for (17000 > 16384 lists): the
    key lists are built by the wave-per-range kernels with global atomics, and the
    gradients still match the oracle and repeat bit for bit."""
    pos = np.arange(17000 - 64, 17000, dtype=np.int32)
    w = tiny_token_workload(seed=71, lengths=(17000,), positions=pos, hq=4, dqk=64, dv=64,
                            hi=4, di=32, topk=37, dtype="bf16")
    _say("token backward global lists")
    d = upload(w)
    idx = csa.dsa_indexer_topk(d["iq"], d["ik"], d["w"], d["layout"], w.topk)
    assert _family(w, d, idx) == "generic"
    dout = np.random.default_rng(71).standard_normal((w.n_q, w.hq, w.dv))
    got = _fwd_bwd(w, d, idx, dout)
    again = _fwd_bwd(w, d, idx, dout)
    for name, a, b in zip(("dq", "dk", "dv"), got[:3], again[:3]):
        assert np.array_equal(a, b), f"{name} differs between two calls"
    _compare(w, idx.cpu().numpy()[:, None, :], got[3], got[:3], TOL["bf16"], "global lists")


def test_backward_is_bitwise_reproducible():
    w = tiny_block_workload(seed=68, layout="all", lengths=(1000, 537), hq=8, hkv=2, d=128,
                            block=64, topk=3, dtype="bf16")
    _say("backward determinism")
    d = upload(w)
    idx = csa.moba_gate_topk(d["q"], d["k"], d["layout"], w.block_size, w.topk)
    dout = np.random.default_rng(68).standard_normal((w.n_q, w.hq, w.dv))
    a = _fwd_bwd(w, d, idx, dout)
    b = _fwd_bwd(w, d, idx, dout)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def _identities(w, dq, dk, dv, dout, lse, label):
    """Key-head sums: sum_j dk[j, g] = 0 and sum_j dv[j, g] = sum of dO over the
    (row, head) pairs of key head g that have keys."""
    group = w.hq // w.hkv
    has = np.isfinite(lse)
    for g in range(w.hkv):
        hs = slice(g * group, (g + 1) * group)
        dsum = (dout[:, hs] * has[:, hs, None]).sum(axis=(0, 1))
        vs = dv[:, g].astype(np.float64).sum(axis=0)
        assert np.abs(vs - dsum).max() <= 1e-3 * max(1.0, np.abs(dv[:, g]).sum(axis=0).max())
        ks = dk[:, g].astype(np.float64).sum(axis=0)
        assert np.abs(ks).max() <= 1e-3 * max(1.0, np.abs(dk[:, g]).sum(axis=0).max())
    _say(label, "key-head sums hold")


def _block_lists(w, idx_np, n_pick=3, max_rows=1500):
    """(g, key start, length, rows) of sampled (key head, block) lists: the block
    holding the last row's position (diagonal mask), the shortest block that is
    selected (a sequence's ragged end, when there is one), and a seeded random
    list; rows = every row that has a head of group g selecting the block."""
    B, G = w.block_size, w.hq // w.hkv
    cu = np.asarray(w.cu_seqlens, np.int64)
    seq = np.asarray(w.q_seq, np.int64)
    pos = np.asarray(w.q_pos, np.int64)
    lo = cu[seq][:, None, None]
    ok = (idx_np >= lo) & (idx_np <= pos[:, None, None]) & ((idx_np - lo) % B == 0)
    starts = []
    for sq in range(len(cu) - 1):
        starts += [(int(a), int(min(B, cu[sq + 1] - a))) for a in range(cu[sq], cu[sq + 1], B)]
    picks = []
    g0 = 0
    last = int(pos[-1])
    picks.append((g0, next(a for a in starts if a[0] <= last < a[0] + a[1])))
    sel_len = sorted((ln, a) for a, ln in starts
                     if ok[:, g0 * G:(g0 + 1) * G][idx_np[:, g0 * G:(g0 + 1) * G] == a].any())
    if sel_len and sel_len[0][0] < B and (g0, (sel_len[0][1], sel_len[0][0])) not in picks:
        picks.append((g0, (sel_len[0][1], sel_len[0][0])))
    rng = np.random.default_rng(9)
    for _ in range(50):
        if len(picks) >= n_pick:
            break
        g = int(rng.integers(w.hkv))
        a = starts[int(rng.integers(len(starts)))]
        hs = slice(g * G, (g + 1) * G)
        nrows = int((ok[:, hs] & (idx_np[:, hs] == a[0])).any(axis=(1, 2)).sum())
        if 0 < nrows <= max_rows and (g, a) not in picks:
            picks.append((g, a))
    out = []
    for g, (a, ln) in picks:
        hs = slice(g * G, (g + 1) * G)
        rows = np.where((ok[:, hs] & (idx_np[:, hs] == a)).any(axis=(1, 2)))[0]
        out.append((g, a, ln, rows))
    return out


def _check_lists(w, idx_np, dout_np, dk, dv, label):
    """dk, dv of whole sampled key blocks against the oracle on every row that
    selects them (restricted to the key head's query heads), spread over worker
    processes."""
    arrays = dict(q=w.q, k=w.k, v=w.value, q_pos=w.q_pos, q_seq=w.q_seq, cu=w.cu_seqlens,
                  idx=idx_np, dout=dout_np)
    with OraclePool(arrays) as pool:
        for g, a, ln, rows in _block_lists(w, idx_np):
            rk, rv = pool.bwd_keys(rows, dict(g=g, a=a, n=ln, mode=w.mode, scale=w.scale,
                                              block_size=w.block_size))
            for name, got, ref in (("dk", dk[a:a + ln, g], rk), ("dv", dv[a:a + ln, g], rv)):
                scale = max(1.0, float(np.abs(ref).max()))
                err = float(np.abs(got - ref).max())
                _say(label, f"{name} of keys [{a}, {a + ln}) head {g} ({len(rows)} rows)",
                     f"err {err:.2e} (scale {scale:.3g})")
                assert err <= TOL["bf16"] * scale


def _check_token_keys(w, idx_np, dout_np, dk, dv, label, n_ranges=2, width=2):
    """dk, dv of sampled runs of `width` consecutive keys against the oracle on
    every row whose selection holds one of them (seeded; keys some row selects)."""
    sel = idx_np[:, 0]
    chosen = np.unique(sel[sel >= 0])
    rng = np.random.default_rng(10)
    arrays = dict(q=w.q, k=w.k, v=w.value, q_pos=w.q_pos, q_seq=w.q_seq, cu=w.cu_seqlens,
                  idx=idx_np, dout=dout_np)
    with OraclePool(arrays) as pool:
        for a in rng.choice(chosen[chosen < w.n_kv - width], n_ranges, replace=False):
            a = int(a)
            rows = np.where(((sel >= a) & (sel < a + width)).any(axis=1))[0]
            rk, rv = pool.bwd_keys(rows, dict(g=0, a=a, n=width, mode=w.mode, scale=w.scale,
                                              block_size=w.block_size))
            for name, got, ref in (("dk", dk[a:a + width, 0], rk), ("dv", dv[a:a + width, 0], rv)):
                scale = max(1.0, float(np.abs(ref).max()))
                err = float(np.abs(got - ref).max())
                _say(label, f"{name} of keys [{a}, {a + width}) ({len(rows)} rows)",
                     f"err {err:.2e} (scale {scale:.3g})")
                assert err <= TOL["bf16"] * scale


@pytest.mark.parametrize("name", ["moba_mha_8k", "moba_gqa_zigzag_32k", "moba_thd_64k",
                                  "dsa_mla_16k"])
def test_full_size_backward(name):
    w = make_workload(name)
    _say("full-size backward", name)
    d = upload(w)
    if w.mode == "block":
        idx = csa.moba_gate_topk(d["q"], d["k"], d["layout"], w.block_size, w.topk)
        idx_np = idx.cpu().numpy()
    else:
        idx = csa.dsa_indexer_topk(d["iq"], d["ik"], d["w"], d["layout"], w.topk)
        idx_np = idx.cpu().numpy()[:, None, :]
    mode = csa.CSA_SEL_BLOCK if w.mode == "block" else csa.CSA_SEL_TOKEN
    assert _family(w, d, idx) == ("block_mfma" if w.mode == "block" else "token_mfma")
    out, lse = csa.sparse_attn_fwd_shard(d["q"], d["k"], d["v"], d["layout"], mode, idx,
                                         block_size=w.block_size, softmax_scale=w.scale,
                                         out_dtype=torch.float32)
    dout_np = (np.random.default_rng(7).standard_normal((w.n_q, w.hq, w.dv))
               .astype(np.float32))
    dout = torch.from_numpy(dout_np).cuda()
    dq = poisoned((w.n_q, w.hq, w.dqk), torch.float32)
    dk = poisoned((w.n_kv, w.hkv, w.dqk), torch.float32)
    dv = poisoned((w.n_kv, w.hkv, w.dv), torch.float32)
    csa.sparse_attn_bwd_shard(d["q"], d["k"], d["v"], d["layout"], mode, idx, out, dout, lse,
                              block_size=w.block_size, softmax_scale=w.scale, dq=dq, dk=dk,
                              dv=dv)
    torch.cuda.synchronize()
    dq, dk, dv = dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()
    lse_np = lse.cpu().numpy()
    for n_, a in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert np.isfinite(a).all(), f"{n_} has unwritten or non-finite elements"
    fam = _family(w, d, idx)
    if fam == "generic":
        # fp32 operands: the key-head sums hold to fp32 rounding
        _identities(w, dq, dk, dv, dout_np.astype(np.float64), lse_np, name)
    elif fam == "token_mfma":
        # bf16 P and dS' operands (see below): sampled keys against the oracle
        _check_token_keys(w, idx_np, dout_np, dk, dv, name)
    else:
        # bf16 P and dS operands: the sums hold only to bf16 rounding (sum_j P_j is
        # 1 within 2^-8), too loose a bar to test; whole key blocks are compared
        _check_lists(w, idx_np, dout_np, dk, dv, name)
    # dq of sampled rows: the oracle's backward restricted to those rows (their dk
    # and dv contributions are ignored here)
    rows = np.unique(np.concatenate([[0, w.n_q - 1, w.n_q // 2],
                                     np.random.default_rng(8).choice(w.n_q, 13, replace=False)]))
    sub_idx = idx_np[rows]
    ref_dq, _, _ = oracle.shard_backward(w.q[rows], w.k, w.value, w.q_pos[rows], w.q_seq[rows],
                                         w.cu_seqlens, w.mode, sub_idx, w.scale, dout_np[rows],
                                         w.block_size)
    err = float(np.abs(dq[rows] - ref_dq).max())
    scale = max(1.0, float(np.abs(ref_dq).max()))
    _say(name, "dq rows", len(rows), "max abs err", f"{err:.3e} (scale {scale:.3g})")
    assert err <= TOL["bf16"] * scale

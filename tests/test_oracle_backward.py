"""Pins for the oracle's backward (gradients with the selection held fixed), CPU only.

``oracle.shard_backward`` is tied to things other than itself:

* central finite differences of the oracle's own forward loss L = sum dO . O,
  element by element, in block mode (GQA, packed sequences, repeated and
  misaligned slots, rows without keys) and token mode (shared index rows,
  per-head index rows, the value aliased to the key's first columns);
* torch float64 autograd through scaled_dot_product_attention on the dense
  special case (every permitted block selected = dense causal attention of the
  shard's queries at their offset against the full key stream);
* zero gradients for rows without keys, and dk/dv zero on keys nobody selected;
* a planted mistake (the softmax Jacobian without its subtraction) that the
  finite differences reject.
"""

import numpy as np
import pytest
import torch

import oracle
from csa_inputs import tiny_block_workload, tiny_token_workload


def _moba_idx(w):
    gate = oracle.gate_scores(w.q, w.k, w.q_pos, w.q_seq, w.cu_seqlens, w.block_size)
    return oracle.select_blocks(gate, w.topk)


def _f64(w):
    return (w.q.astype(np.float64), w.k.astype(np.float64), w.value.astype(np.float64))


def _fd_check(w, idx, dout, q, k, v, n_probe=40, seed=0, eps=1e-6, alias=False):
    """Central differences on random elements of q, k and v against the oracle."""
    dq, dk, dv = oracle.shard_backward(q, k, v, w.q_pos, w.q_seq, w.cu_seqlens, w.mode, idx,
                                       w.scale, dout, w.block_size)
    rng = np.random.default_rng(seed)

    def L(q_, k_, v_):
        return oracle.loss(q_, k_, v_, w.q_pos, w.q_seq, w.cu_seqlens, w.mode, idx, w.scale,
                           dout, w.block_size)

    targets = [("q", q, dq), ("k", k, dk)] + ([] if alias else [("v", v, dv)])
    for name, arr, grad in targets:
        for _ in range(n_probe):
            e = tuple(int(rng.integers(0, s)) for s in arr.shape)
            plus, minus = arr.copy(), arr.copy()
            plus[e] += eps
            minus[e] -= eps
            if alias:  # the value is a view of the key's first columns
                args_p = (q, plus, plus[..., :w.dv]) if name == "k" else (plus, k, k[..., :w.dv])
                args_m = (q, minus, minus[..., :w.dv]) if name == "k" else (minus, k, k[..., :w.dv])
            else:
                args_p = {"q": (plus, k, v), "k": (q, plus, v), "v": (q, k, plus)}[name]
                args_m = {"q": (minus, k, v), "k": (q, minus, v), "v": (q, k, minus)}[name]
            num = (L(*args_p) - L(*args_m)) / (2 * eps)
            ana = grad[e]
            if alias and name == "k" and e[2] < w.dv:
                ana = ana + dv[e]  # the shared tensor feeds the value too
            assert abs(num - ana) <= 1e-6 * max(1.0, abs(num)), (name, e, num, ana)
    return dq, dk, dv


@pytest.mark.parametrize("seed,layout,lengths,hq,hkv,topk", [
    (0, "contiguous", (40, 24), 4, 2, 2),
    (1, "zigzag", (64,), 4, 4, 3),
    (2, "all", (13, 30, 21), 6, 2, 1),
])
def test_block_backward_matches_finite_differences(seed, layout, lengths, hq, hkv, topk):
    w = tiny_block_workload(seed=seed, layout=layout, lengths=lengths, hq=hq, hkv=hkv, d=8,
                            block=8, topk=topk)
    idx = _moba_idx(w)
    dout = np.random.default_rng(seed + 100).standard_normal((w.n_q, w.hq, w.dv))
    _fd_check(w, idx, dout, *_f64(w), seed=seed)


def test_caller_slots_backward_matches_finite_differences():
    """Repeated, misaligned, future, out-of-range and pad slots; rows without keys."""
    w = tiny_block_workload(seed=4, layout="all", lengths=(20, 28, 16), hq=4, hkv=2, d=8,
                            block=8, topk=2)
    rng = np.random.default_rng(4)
    idx = rng.integers(-3, w.n_kv + 3, size=(w.n_q, w.hq, 5)).astype(np.int32)
    for i in range(w.n_q):
        lo = int(w.cu_seqlens[w.q_seq[i]])
        idx[i, :, 0] = lo + w.block_size * rng.integers(0, 3, size=w.hq)
    idx[::3, :, 1] = idx[::3, :, 0]  # a repeated slot counts twice
    q_seq = w.q_seq.copy()
    q_seq[3] = 7  # no such sequence: no keys
    w.q_seq = q_seq
    dout = rng.standard_normal((w.n_q, w.hq, w.dv))
    dq, dk, dv = _fd_check(w, idx, dout, *_f64(w), seed=4)
    assert not dq[3].any()


@pytest.mark.parametrize("shared", [True, False])
def test_token_backward_matches_finite_differences(shared):
    w = tiny_token_workload(seed=6, lengths=(30, 20), hq=4, dqk=12, dv=8, hi=3, di=8, topk=6)
    rng = np.random.default_rng(6)
    heads = 1 if shared else w.hq
    idx = rng.integers(-2, w.n_kv + 2, size=(w.n_q, heads, 7)).astype(np.int32)
    dout = rng.standard_normal((w.n_q, w.hq, w.dv))
    q, k, _ = _f64(w)
    # the value is the first Dv columns of the key (absorbed MLA): differences of
    # the shared tensor see dk + dv on those columns
    _fd_check(w, idx, dout, q, k, k[..., :w.dv], seed=7, alias=True)


def test_dense_special_case_matches_torch_autograd():
    """All permitted blocks selected: the gradients of dense causal attention of the
    shard's queries at their global offset, from torch float64 autograd."""
    w = tiny_block_workload(seed=9, layout="contiguous", cp=4, rank=2, lengths=(64,), hq=4,
                            hkv=2, d=8, block=8, topk=8)
    idx = _moba_idx(w)
    rng = np.random.default_rng(9)
    dout = rng.standard_normal((w.n_q, w.hq, w.dv))
    q, k, v = _f64(w)
    dq, dk, dv = oracle.shard_backward(q, k, v, w.q_pos, w.q_seq, w.cu_seqlens, "block", idx,
                                       w.scale, dout, w.block_size)
    group = w.hq // w.hkv
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    kr = tk.repeat_interleave(group, dim=1).permute(1, 0, 2)   # [Hq, n_kv, D]
    vr = tv.repeat_interleave(group, dim=1).permute(1, 0, 2)
    mask = torch.tensor(np.arange(w.n_kv)[None, :] <= w.q_pos[:, None])  # shifted causal
    out = torch.nn.functional.scaled_dot_product_attention(
        tq.permute(1, 0, 2), kr, vr, attn_mask=mask, scale=w.scale)
    (out.permute(1, 0, 2) * torch.tensor(dout)).sum().backward()
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-12)
    # keys after the shard's last position get nothing
    assert not dk[w.q_pos.max() + 1:].any() and not dv[w.q_pos.max() + 1:].any()


def test_planted_jacobian_mistake_is_caught():
    """A backward that drops the softmax Jacobian's subtraction disagrees with the
    finite differences of the forward."""
    w = tiny_block_workload(seed=12, layout="all", lengths=(32,), hq=2, hkv=2, d=8, block=8,
                            topk=2)
    idx = _moba_idx(w)
    rng = np.random.default_rng(12)
    dout = rng.standard_normal((w.n_q, w.hq, w.dv))
    q, k, v = _f64(w)
    i, h = 20, 1
    keys = oracle.selected_keys("block", idx[i, h], (0, int(w.q_pos[i]), 32), w.block_size)
    kmat, vmat = k[keys, h], v[keys, h]
    x = w.scale * (kmat @ q[i, h])
    p = np.exp(x - x.max())
    p /= p.sum()
    wrong = w.scale * ((p * (vmat @ dout[i, h])) @ kmat)   # no "- sum P dP"
    dq, _, _ = oracle.shard_backward(q, k, v, w.q_pos, w.q_seq, w.cu_seqlens, "block", idx,
                                     w.scale, dout, w.block_size)
    eps = 1e-6
    num = np.zeros(w.dqk)
    for c in range(w.dqk):
        qp, qm = q.copy(), q.copy()
        qp[i, h, c] += eps
        qm[i, h, c] -= eps
        num[c] = (oracle.loss(qp, k, v, w.q_pos, w.q_seq, w.cu_seqlens, "block", idx, w.scale,
                              dout, w.block_size) -
                  oracle.loss(qm, k, v, w.q_pos, w.q_seq, w.cu_seqlens, "block", idx, w.scale,
                              dout, w.block_size)) / (2 * eps)
    np.testing.assert_allclose(dq[i, h], num, rtol=1e-6, atol=1e-8)
    assert np.abs(wrong - num).max() > 1e-3

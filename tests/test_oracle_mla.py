"""Pins for the oracle's absorbed-MLA value up-projection (CPU only).

Passage: Megatron-LM PR #3674, "[1/2] Enable DSA CP, THD with absorbed MLA" -
the earlier PR description quoted there (the value up-projection is applied
after sparse attention) and the review summary's sequence diagram (an einsum
with up_v_weight after the sparse attention).
"""

import numpy as np

import oracle


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_identity_slice_is_exact():
    # w[h] = [I | 0]: each head keeps the first Dv latent channels unchanged
    rng = np.random.default_rng(1)
    n_q, hq, dl, dv = 7, 3, 40, 12
    o = _rand(rng, n_q, hq, dl)
    w = np.zeros((hq, dv, dl))
    for h in range(hq):
        w[h, :, :dv] = np.eye(dv)
    out = oracle.v_up_proj(o, w)
    assert out.shape == (n_q, hq, dv)
    assert np.array_equal(out, o[:, :, :dv])


def test_one_hot_rows_pick_channels_per_head():
    # row d of head h selects latent channel perm_h[d]: a per-head gather
    rng = np.random.default_rng(2)
    n_q, hq, dl, dv = 5, 4, 24, 6
    o = _rand(rng, n_q, hq, dl)
    w = np.zeros((hq, dv, dl))
    perms = [rng.permutation(dl)[:dv] for _ in range(hq)]
    for h in range(hq):
        w[h, np.arange(dv), perms[h]] = 1.0
    out = oracle.v_up_proj(o, w)
    for h in range(hq):
        assert np.array_equal(out[:, h, :], o[:, h, perms[h]])


def test_ones_weight_is_channel_sum():
    rng = np.random.default_rng(3)
    o = _rand(rng, 6, 2, 33)
    out = oracle.v_up_proj(o, np.ones((2, 4, 33)))
    np.testing.assert_allclose(out, np.repeat(o.sum(axis=2, keepdims=True), 4, axis=2),
                               rtol=1e-13, atol=1e-13)


def test_after_attention_equals_attention_over_projected_values():
    # Up-projecting the attention output of the latent values equals attending
    # over each head's up-projected values (the softmax weights do not depend
    # on the values).  One latent key head, as in absorbed MLA; the projected
    # values differ per query head, so they are attended with the key head
    # repeated per query head.
    rng = np.random.default_rng(4)
    n_kv, n_q, hq, dqk, dl, dv = 40, 9, 3, 20, 16, 5
    k = _rand(rng, n_kv, 1, dqk)
    c = k[:, :, :dl]  # the value is the latent part of the key
    q = _rand(rng, n_q, hq, dqk)
    w = _rand(rng, hq, dv, dl)
    q_pos = np.arange(n_kv - n_q, n_kv, dtype=np.int32)
    q_seq = np.zeros(n_q, np.int32)
    cu = np.array([0, n_kv], np.int32)
    idx = np.stack([rng.permutation(n_kv)[:12] for _ in range(n_q)])[:, None, :]
    scale = 1.0 / np.sqrt(dqk)
    o_lat, lse_a = oracle.shard_forward(q, k, c, q_pos, q_seq, cu, "token", idx, scale)
    up = oracle.v_up_proj(o_lat, w)
    k_rep = np.repeat(k, hq, axis=1)
    v_proj = np.einsum("jc,hdc->jhd", c[:, 0, :], w)
    direct, lse_b = oracle.shard_forward(q, k_rep, v_proj, q_pos, q_seq, cu, "token", idx, scale)
    np.testing.assert_allclose(up, direct, rtol=1e-11, atol=1e-12)
    # the two runs group the heads differently (one key head against three), so
    # their fp64 logits are summed in different orders
    np.testing.assert_allclose(lse_a, lse_b, rtol=1e-14, atol=1e-14)

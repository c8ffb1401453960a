"""Pins for the oracle's chunk summaries, merge and finalize (CPU only).

Passage: "Context parallel attention: exchange keys and merge softmax globally",
paragraphs on the chunk summary / merge and on the neutral summary.
"""

import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "two_chunk_merge.txt")


def _golden():
    vals = {}
    with open(GOLDEN) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            name, *nums = line.split()
            vals[name] = [float(x) for x in nums]
    return vals


def test_two_chunk_closed_form():
    g = _golden()
    va = np.array(g["a_values"])[:, None]
    vb = np.array(g["b_values"])[:, None]
    a = oracle.summary(g["a_logits"], va)
    b = oracle.summary(g["b_logits"], vb)
    assert a[0] == pytest.approx(g["a_m"][0], rel=1e-15)
    assert a[1] == pytest.approx(g["a_l"][0], rel=1e-15)
    assert a[2][0] == pytest.approx(g["a_z"][0], rel=1e-15)
    assert b[1] == pytest.approx(g["b_l"][0], rel=1e-15)
    s = oracle.merge(a, b)
    assert s[0] == pytest.approx(g["merged_m"][0], rel=1e-15)
    assert s[1] == pytest.approx(g["merged_l"][0], rel=1e-15)
    assert s[2][0] == pytest.approx(g["merged_z"][0], rel=1e-15)
    o, lse = oracle.finalize(s)
    assert o[0] == pytest.approx(47.0 / 7.0, rel=1e-15)
    assert o[0] == pytest.approx(g["o"][0], rel=1e-15)
    assert lse == pytest.approx(math.log(7.0), rel=1e-15)
    # merging in the other order reaches the same numbers
    s2 = oracle.merge(b, a)
    assert s2[1] == pytest.approx(1.75, rel=1e-15)
    assert s2[2][0] == pytest.approx(11.75, rel=1e-15)


def test_large_offset_no_overflow():
    # +800 on every logit: exp(800) overflows float64, the rescaled merge does not
    a = oracle.summary([800.0, 800.0 + math.log(2.0)], np.array([[1.0], [3.0]]))
    b = oracle.summary([800.0 + math.log(4.0)], np.array([[10.0]]))
    o, lse = oracle.finalize(oracle.merge(a, b))
    assert np.isfinite(o).all()
    assert o[0] == pytest.approx(47.0 / 7.0, rel=1e-13)
    assert lse == pytest.approx(800.0 + math.log(7.0), rel=1e-15)


def test_neutral_is_identity_and_no_nan():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(7)
    v = rng.standard_normal((7, 3))
    s = oracle.summary(x, v)
    neutral = oracle.summary([], np.zeros((0, 3)))
    assert neutral[0] == -np.inf and neutral[1] == 0.0 and not neutral[2].any()
    for merged in (oracle.merge(s, neutral), oracle.merge(neutral, s)):
        assert merged[0] == s[0]
        assert merged[1] == s[1]
        assert np.array_equal(merged[2], s[2])
    nn = oracle.merge(neutral, neutral)
    assert nn[0] == -np.inf and nn[1] == 0.0
    assert not np.isnan(nn[2]).any()
    o, lse = oracle.finalize(nn)
    assert lse == -np.inf and not o.any() and not np.isnan(o).any()


def test_merge_equals_union_softmax():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(50) * 3
    v = rng.standard_normal((50, 4))
    for cut in (1, 17, 49):
        a = oracle.summary(x[:cut], v[:cut])
        b = oracle.summary(x[cut:], v[cut:])
        m, ell, z = oracle.merge(a, b)
        m2, l2, z2 = oracle.summary(x, v)
        assert m == m2
        assert ell == pytest.approx(l2, rel=1e-14)
        np.testing.assert_allclose(z, z2, rtol=1e-13, atol=1e-14)
    # and the finalized union equals a direct softmax-weighted average
    w = np.exp(x - x.max())
    direct = (w / w.sum()) @ v
    o, _ = oracle.finalize(oracle.summary(x, v))
    np.testing.assert_allclose(o, direct, rtol=1e-13, atol=1e-14)


def test_merge_parts_matches_pairwise_and_single_pass():
    rng = np.random.default_rng(2)
    P, R, dv = 4, 6, 3
    xs = [[rng.standard_normal(rng.integers(0, 5)) for _ in range(R)] for _ in range(P)]
    vs = [[rng.standard_normal((len(xs[p][r]), dv)) for r in range(R)] for p in range(P)]
    m = np.zeros((P, R))
    ell = np.zeros((P, R))
    z = np.zeros((P, R, dv))
    for p in range(P):
        for r in range(R):
            m[p, r], ell[p, r], z[p, r] = oracle.summary(xs[p][r], vs[p][r])
    mo, lo, zo = oracle.merge_parts(m, ell, z)
    for r in range(R):
        x_all = np.concatenate([xs[p][r] for p in range(P)])
        v_all = np.concatenate([vs[p][r] for p in range(P)])
        m2, l2, z2 = oracle.summary(x_all, v_all)
        assert mo[r] == m2
        assert lo[r] == pytest.approx(l2, rel=1e-14)
        np.testing.assert_allclose(zo[r], z2, rtol=1e-13, atol=1e-14)


def test_planted_sign_error_is_caught():
    """A merge that rescales with exp(m - m_X) instead of exp(m_X - m) fails the pin."""
    def bad_merge(a, b):
        ma, la, za = a
        mb, lb, zb = b
        m = max(ma, mb)
        wa = 0.0 if ma == -np.inf else np.exp(m - ma)
        wb = 0.0 if mb == -np.inf else np.exp(m - mb)
        return m, wa * la + wb * lb, wa * za + wb * zb

    _check_with(oracle.merge)
    with pytest.raises(AssertionError):
        _check_with(bad_merge)


def _check_with(merge_fn):
    g = _golden()
    a = oracle.summary(g["a_logits"], np.array(g["a_values"])[:, None])
    b = oracle.summary(g["b_logits"], np.array(g["b_values"])[:, None])
    s = merge_fn(a, b)
    assert s[2][0] == pytest.approx(g["merged_z"][0], rel=1e-12)

"""Pins for the routing oracle (CPU only)."""
import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle.route import route_topk, route_topk_brute


def test_golden_small(golden):
    g = golden("route_small.txt")
    logits = np.array([[float(v) for v in r] for r in g["logits"]], dtype=np.float32)
    idx, w = route_topk(logits, 2)
    assert idx.tolist() == [[int(v) for v in r] for r in g["idx"]]
    lg = lambda a: 1.0 / (1.0 + math.exp(-a))
    closed = np.array([[0.5, 0.5], [lg(1.0), lg(-1.0)]], dtype=np.float32)
    np.testing.assert_allclose(w, closed, rtol=1.2e-7, atol=0)
    bi, bw = route_topk_brute(logits, 2)
    assert np.array_equal(bi, idx)
    np.testing.assert_allclose(bw, w, rtol=1.2e-7, atol=0)


@settings(max_examples=60, deadline=None)
@given(st.integers(1, 12), st.sampled_from([1, 2, 3, 4, 8, 16]), st.data())
def test_numpy_matches_brute_force(n, e, data):
    k = data.draw(st.integers(1, e))
    renorm = data.draw(st.booleans())
    seed = data.draw(st.integers(0, 2**31))
    rng = np.random.default_rng(seed)
    # few distinct values -> many ties; include signed zeros
    pool = np.array([-2.0, -0.5, -0.0, 0.0, 0.5, 1.0, 3.0], dtype=np.float32)
    logits = pool[rng.integers(0, pool.size, (n, e))] if data.draw(st.booleans()) \
        else rng.standard_normal((n, e)).astype(np.float32)
    i1, w1 = route_topk(logits, k, renorm)
    i0, w0 = route_topk_brute(logits, k, renorm)
    assert np.array_equal(i0, i1)
    np.testing.assert_allclose(w1, w0, rtol=2e-7, atol=0)


def test_all_equal_logits():
    for e, k in ((8, 2), (256, 8), (64, 64)):
        logits = np.full((3, e), 0.25, dtype=np.float32)
        idx, w = route_topk(logits, k)
        assert (idx == np.arange(k)).all()
        assert (w == np.float32(1.0 / k)).all()


def test_descending_ramp_and_signed_zero():
    logits = -np.arange(16, dtype=np.float32)[None, :].repeat(2, 0)
    idx, _ = route_topk(logits, 5)
    assert (idx == np.arange(5)).all()
    z = np.array([[-0.0, 0.0, -1.0], [0.0, -0.0, -1.0]], dtype=np.float32)
    idx, w = route_topk(z, 2)
    assert idx.tolist() == [[0, 1], [0, 1]]
    assert (w == np.float32(0.5)).all()


def test_k2_logistic_closed_form():
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((500, 8)).astype(np.float32)
    idx, w = route_topk(logits, 2)
    l0 = np.take_along_axis(logits, idx[:, :1], 1)[:, 0].astype(np.float64)
    l1 = np.take_along_axis(logits, idx[:, 1:2], 1)[:, 0].astype(np.float64)
    expect = 1.0 / (1.0 + np.exp(-(l0 - l1)))
    np.testing.assert_allclose(w[:, 0], expect, rtol=1.2e-7)
    np.testing.assert_allclose(w[:, 1], 1.0 - expect, rtol=1e-6)


def test_full_softmax_when_k_equals_e():
    rng = np.random.default_rng(4)
    logits = rng.standard_normal((50, 16)).astype(np.float32)
    idx, w = route_topk(logits, 16, renormalize=False)
    # weights in expert order equal scipy's softmax (a library routine)
    from scipy.special import softmax
    back = np.empty_like(w)
    np.put_along_axis(back, idx.astype(np.int64), w, 1)
    np.testing.assert_allclose(back, softmax(logits.astype(np.float64), axis=1), rtol=1e-6)


def test_weight_invariants():
    rng = np.random.default_rng(7)
    logits = rng.standard_normal((2000, 256)).astype(np.float32)
    for renorm in (True, False):
        idx, w = route_topk(logits, 8, renorm)
        assert (np.diff(w, axis=1) <= 0).all()
        sel = np.take_along_axis(logits, idx.astype(np.int64), 1)
        assert (np.diff(sel, axis=1) <= 0).all()
        # the selected set is the k largest
        kth = np.sort(logits, axis=1)[:, -8]
        assert (sel[:, -1] == kth).all()
        s = w.astype(np.float64).sum(1)
        if renorm:
            np.testing.assert_allclose(s, 1.0, atol=8 * 2**-24)
        else:
            assert (s < 1.0 + 1e-6).all()
    # each row's indices are distinct
    assert all(len(set(r)) == 8 for r in idx.tolist())


def test_rejects_bad_k():
    with pytest.raises(ValueError):
        route_topk(np.zeros((2, 4), np.float32), 5)

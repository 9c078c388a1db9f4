"""Pins for the dispatch oracle (CPU only)."""
from collections import Counter

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import dispatch as od


def _ints(row):
    return [int(v) for v in row]


def test_golden_small(golden):
    g = golden("dispatch_small.txt")
    idx = np.array([_ints(r) for r in g["idx"]], dtype=np.int32)
    assert od.expert_counts(idx, 4).tolist() == _ints(g["expert_counts"])
    offs = od.expert_offsets(od.expert_counts(idx, 4))
    assert offs.tolist() == _ints(g["expert_offsets"])
    for name, sorted_, nseg in (("sorted", True, 1), ("unsorted_g1", False, 1),
                                ("unsorted_g2", False, 2)):
        for impl in (od.permutation, od.permutation_brute):
            src, dst, rexp = impl(idx, 4, nseg, sorted_)
            assert src.tolist() == _ints(g[name + ".src_pair"]), (name, impl)
            assert dst.tolist() == _ints(g[name + ".dst_pos"]), (name, impl)
            assert rexp.tolist() == _ints(g[name + ".row_expert"]), (name, impl)
    assert od.segment_offsets(offs, 4, 2).tolist() == _ints(g["segment_offsets_g2"])
    x = np.array([[10 * t, 10 * t + 1] for t in range(4)], dtype=np.int32)
    src, _, _ = od.permutation(idx, 4, 1, True)
    rows = od.gather_rows(x, src, 2)
    assert (rows[:, 0] // 10).tolist() == _ints(g["sorted.row_tokens"])


@settings(max_examples=80, deadline=None)
@given(st.integers(0, 24), st.sampled_from([(1, 1), (4, 1), (4, 2), (8, 1), (8, 4), (16, 8)]),
       st.integers(1, 4), st.booleans(), st.integers(0, 2**31))
def test_argsort_form_matches_brute(n, eg, k, sorted_, seed):
    e, g = eg
    k = min(k, e)
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, e, (n, k)).astype(np.int32)   # duplicates within a token allowed
    a = od.permutation(idx, e, g, sorted_)
    b = od.permutation_brute(idx, e, g, sorted_)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def _random_idx(rng, n, e, k):
    return np.stack([rng.permutation(e)[:k] for _ in range(n)]).astype(np.int32)


@pytest.mark.parametrize("n,e,k,g", [(16, 8, 2, 1), (300, 256, 8, 8), (1000, 64, 4, 4), (1, 8, 8, 2)])
def test_invariants(n, e, k, g):
    rng = np.random.default_rng(n + e)
    idx = _random_idx(rng, n, e, k)
    counts = od.expert_counts(idx, e)
    assert counts.sum() == n * k
    c = Counter(idx.ravel().tolist())
    assert counts.tolist() == [c.get(i, 0) for i in range(e)]
    offs = od.expert_offsets(counts)
    assert offs[0] == 0 and offs[-1] == n * k and (np.diff(offs) >= 0).all()
    segs = od.segment_offsets(offs, e, g)
    assert segs.size == g + 1 and segs[-1] == n * k
    results = {}
    for sorted_ in (True, False):
        src, dst, rexp = od.permutation(idx, e, g, sorted_)
        results[sorted_] = (src, dst, rexp)
        nk = n * k
        assert np.array_equal(np.sort(src), np.arange(nk))          # a permutation
        assert np.array_equal(dst[src], np.arange(nk))              # dst is its inverse
        assert np.array_equal(src[dst], np.arange(nk))
        assert np.array_equal(rexp, idx.ravel()[src])
        key = rexp if sorted_ else rexp // (e // g)
        assert (np.diff(key) >= 0).all()                            # grouped by bucket
        for b in np.unique(key):                                    # stable inside a bucket
            assert (np.diff(src[key == b]) > 0).all()
        if sorted_:
            for ee in range(e):                                     # expert blocks at offsets
                assert (rexp[offs[ee]:offs[ee + 1]] == ee).all()
        for gg in range(g):                                         # segment blocks at offsets
            blk = rexp[segs[gg]:segs[gg + 1]] // (e // g)
            assert (blk == gg).all()
    # sorted with G segments is the same permutation as sorted with one
    s1 = od.permutation(idx, e, 1, True)
    for u, v in zip(results[True], s1):
        assert np.array_equal(u, v)
    # unsorted, one segment: identity
    src, dst, _ = od.permutation(idx, e, 1, False)
    assert np.array_equal(src, np.arange(n * k)) and np.array_equal(dst, np.arange(n * k))


def test_rows_gather_equals_scatter_and_round_trip():
    rng = np.random.default_rng(1)
    n, e, k, d = 40, 16, 4, 24
    idx = _random_idx(rng, n, e, k)
    x = rng.integers(0, 2**16, (n, d)).astype(np.uint16)
    src, dst, _ = od.permutation(idx, e, 1, True)
    rows = od.gather_rows(x, src, k)
    assert np.array_equal(rows, od.scatter_rows(x, dst, k))
    # inverse restores the order: rows[dst_pos[t*k+j]] is token t's row
    back = rows[dst].reshape(n, k, d)
    assert all(np.array_equal(back[:, j], x) for j in range(k))


def test_resolve_sorted():
    assert od.resolve_sorted(1, 1, 256) is True
    assert od.resolve_sorted(0, 10**6, 256) is False
    assert od.resolve_sorted(-1, 256, 256) is False      # (256-1)//256 == 0
    assert od.resolve_sorted(-1, 257, 256) is True       # (257-1)//256 == 1
    assert od.resolve_sorted(-1, 128, 256) is False
    assert od.resolve_sorted(-1, 4096, 256) is True
    assert od.resolve_sorted(-1, 1, 1) is False
    assert od.resolve_sorted(-1, 2, 1) is True
    assert od.resolve_sorted(-1, 5, 0) is True           # guard: cutoff <= 0 always sorts
    with pytest.raises(ValueError):
        od.resolve_sorted(2, 5, 1)

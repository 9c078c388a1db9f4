"""Pins for the grouped SwiGLU oracle (CPU only)."""
import math

import numpy as np

from oracle import codecs, dispatch as od
from oracle.swiglu import (_bf16_round_py, grouped_swiglu, silu, swiglu_brute, swiglu_combine,
                           swiglu_hidden, swiglu_rows, swiglu_rows_f64)


def _bf16(a):
    return codecs.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def test_silu_closed_forms():
    a = np.linspace(-30, 30, 601)
    assert silu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(silu(a) - silu(-a), a, rtol=1e-14, atol=1e-14)
    assert abs(silu(np.array([40.0]))[0] - 40.0) < 1e-12
    np.testing.assert_allclose(silu(np.array([1.0])), [1.0 / (1.0 + np.exp(-1.0))], rtol=1e-15)


def test_rows_match_pure_python_brute_force():
    rng = np.random.default_rng(0)
    e, f, d = 3, 6, 5
    wg, wu = _bf16(rng.standard_normal((e, f, d)) * 0.5), _bf16(rng.standard_normal((e, f, d)) * 0.5)
    wd = _bf16(rng.standard_normal((e, d, f)) * 0.5)
    rows = _bf16(rng.standard_normal((7, d)))
    experts = np.array([2, 0, 2, 1, 1, 0, 2])
    got = codecs.bf16_bits_to_f32(swiglu_rows(rows, experts, wg, wu, wd))
    dec = lambda b: codecs.bf16_bits_to_f32(b).astype(np.float64).tolist()
    for p, ex in enumerate(experts):
        ref = swiglu_brute(dec(rows[p]), dec(wg[ex]), dec(wu[ex]), dec(wd[ex]))
        ref_b = codecs.bf16_bits_to_f32(codecs.f64_to_bf16_bits(np.array(ref)))
        # h is rounded to bf16 on both sides; a 1-ulp flip of one h element can
        # move y by much less than a bf16 ulp, so compare within one ulp
        assert np.all(np.abs(got[p] - ref_b) <= np.abs(ref_b) * 2**-7 + 1e-30), p


def test_hidden_matches_brute_force_and_feeds_the_down_product():
    """h on its own: each element against a pure-Python fsum of the gate and
    up dot products, silu by math.exp and the scaling RNE of swiglu_brute; then
    h times W_down (float64) rounded once must be swiglu_rows exactly."""
    rng = np.random.default_rng(7)
    e, f, d = 3, 9, 6
    wg, wu = _bf16(rng.standard_normal((e, f, d)) * 0.5), _bf16(rng.standard_normal((e, f, d)) * 0.5)
    wd = _bf16(rng.standard_normal((e, d, f)) * 0.5)
    rows = _bf16(rng.standard_normal((8, d)))
    experts = np.array([1, 2, 0, 1, -1, 2, 2, 0])
    h = swiglu_hidden(rows, experts, wg, wu)
    assert h.shape == (8, f)
    assert (h[4] == 0).all()                            # bad id: no row
    dec = lambda b: codecs.bf16_bits_to_f32(b).astype(np.float64).tolist()
    for p, ex in enumerate(experts):
        if ex < 0:
            continue
        r = dec(rows[p])
        for i in range(f):
            g = math.fsum(a * b for a, b in zip(dec(wg[ex][i]), r))
            u = math.fsum(a * b for a, b in zip(dec(wu[ex][i]), r))
            want = _bf16_round_py(g / (1.0 + math.exp(-g)) * u)
            assert float(codecs.bf16_bits_to_f32(h[p:p + 1, i])[0]) == want, (p, i)
    ok = experts >= 0
    hf = codecs.bf16_bits_to_f32(h[ok]).astype(np.float64)
    y = np.stack([hf[i] @ codecs.bf16_bits_to_f32(wd[ex]).astype(np.float64).T
                  for i, ex in enumerate(experts[ok])])
    assert np.array_equal(codecs.f64_to_bf16_bits(y), swiglu_rows(rows[ok], experts[ok], wg, wu, wd))


def test_unit_case_two_rows_on_one_expert():
    # the gather_mm shape of the MLX test named gather_mm_e4_i64_o128_sorted:
    # E=4, in=64, out=128, both rows on expert 3 (a single segment)
    rng = np.random.default_rng(1)
    e, d, f = 4, 64, 128
    wg, wu = _bf16(rng.standard_normal((e, f, d)) * 0.1), _bf16(rng.standard_normal((e, f, d)) * 0.1)
    wd = _bf16(rng.standard_normal((e, d, f)) * 0.1)
    rows = _bf16(rng.standard_normal((2, d)))
    offs = np.array([0, 0, 0, 0, 2])
    y = grouped_swiglu(rows, offs, wg, wu, wd)
    y3 = swiglu_rows(rows, np.array([3, 3]), wg, wu, wd)
    assert np.array_equal(y, y3)
    # experts 0..2 are empty and produce no rows; a different expert changes y
    assert not np.array_equal(y, swiglu_rows(rows, np.array([0, 0]), wg, wu, wd))


def test_layout_invariance():
    rng = np.random.default_rng(2)
    n, e, k, d, f = 24, 4, 2, 8, 12
    wg, wu = _bf16(rng.standard_normal((e, f, d)) * 0.3), _bf16(rng.standard_normal((e, f, d)) * 0.3)
    wd = _bf16(rng.standard_normal((e, d, f)) * 0.3)
    x = _bf16(rng.standard_normal((n, d)))
    idx = np.stack([rng.permutation(e)[:k] for _ in range(n)]).astype(np.int32)
    per_pair = {}
    for sorted_ in (True, False):
        src, dst, rexp = od.permutation(idx, e, 1, sorted_)
        rows = od.gather_rows(x, src, k)
        y = swiglu_rows(rows, rexp, wg, wu, wd)
        per_pair[sorted_] = y[dst]          # back to pair order
    assert np.array_equal(per_pair[True], per_pair[False])


def _fused_case(seed=3, n=5, k=3, e=4, d=6, f=7):
    rng = np.random.default_rng(seed)
    wg, wu = _bf16(rng.standard_normal((e, f, d)) * 0.4), _bf16(rng.standard_normal((e, f, d)) * 0.4)
    wd = _bf16(rng.standard_normal((e, d, f)) * 0.4)
    rows = _bf16(rng.standard_normal((n * k, d)))
    experts = rng.integers(0, e, n * k)
    row_pair = rng.permutation(n * k)                   # rows in a shuffled layout
    tw = rng.uniform(0.05, 1.0, (n, k)).astype(np.float32)
    return rows, experts, row_pair, tw, k, (wg, wu, wd)


def test_fused_combine_matches_pure_python_brute_force():
    rows, experts, row_pair, tw, k, w = _fused_case()
    out0 = np.arange(5 * 6, dtype=np.float64).reshape(5, 6) * 0.25
    got = swiglu_combine(rows, experts, row_pair, tw, k, *w, out0=out0)
    dec = lambda b: codecs.bf16_bits_to_f32(b).astype(np.float64).tolist()
    n = tw.shape[0]
    for t in range(n):
        for i in range(6):
            terms = [out0[t, i]]
            for j in range(k):
                r = [rr for rr in range(len(row_pair)) if row_pair[rr] == t * k + j][0]
                ex = experts[r]
                y = swiglu_brute(dec(rows[r]), dec(w[0][ex]), dec(w[1][ex]), dec(w[2][ex]))
                terms.append(float(tw[t, j]) * y[i])
            ref = math.fsum(terms)
            # h is rounded to bf16 on both sides (a tie-side flip moves y by far
            # less than this); the sums are otherwise exact up to float64
            assert abs(got[t, i] - ref) <= 1e-3 * math.fsum(abs(v) for v in terms) + 1e-12, (t, i)


def test_fused_combine_k1_unit_weights_is_the_unrounded_ffn():
    rng = np.random.default_rng(4)
    e, d, f, n = 3, 5, 4, 6
    wg, wu = _bf16(rng.standard_normal((e, f, d))), _bf16(rng.standard_normal((e, f, d)))
    wd = _bf16(rng.standard_normal((e, d, f)))
    rows = _bf16(rng.standard_normal((n, d)))
    experts = rng.integers(0, e, n)
    got = swiglu_combine(rows, experts, np.arange(n), np.ones((n, 1), np.float32), 1, wg, wu, wd)
    assert np.array_equal(got, swiglu_rows_f64(rows, experts, wg, wu, wd))
    # and rounding it gives the rounded FFN rows
    assert np.array_equal(codecs.f64_to_bf16_bits(got), swiglu_rows(rows, experts, wg, wu, wd))


def test_fused_combine_invariant_under_row_shuffle_and_skips_bad_ids():
    rows, experts, row_pair, tw, k, w = _fused_case(seed=5)
    a = swiglu_combine(rows, experts, row_pair, tw, k, *w)
    perm = np.random.default_rng(6).permutation(len(row_pair))
    b = swiglu_combine(rows[perm], experts[perm], row_pair[perm], tw, k, *w)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-13)
    bad = experts.copy()
    bad[0] = 99                                          # this row takes no part
    c = swiglu_combine(rows, bad, row_pair, tw, k, *w)
    t0 = row_pair[0] // k
    others = np.arange(tw.shape[0]) != t0
    assert np.array_equal(c[others], a[others]) and not np.allclose(c[t0], a[t0])


from hypothesis import given, settings, strategies as st


@settings(max_examples=40, deadline=None)
@given(st.integers(1, 4), st.integers(1, 3), st.integers(1, 3), st.integers(1, 5), st.integers(1, 5),
       st.integers(0, 2**32 - 1))
def test_fused_combine_brute_force_sweep(n, k, e, d, f, seed):
    """Random small shapes, rows in a shuffled layout, some rows with an expert
    outside [0, E): the fused combine against a pure-Python evaluation that
    looks each pair's row up by scanning the rows."""
    rng = np.random.default_rng(seed)
    wg, wu = _bf16(rng.standard_normal((e, f, d)) * 0.5), _bf16(rng.standard_normal((e, f, d)) * 0.5)
    wd = _bf16(rng.standard_normal((e, d, f)) * 0.5)
    rows = _bf16(rng.standard_normal((n * k, d)))
    experts = rng.integers(-1, e + 1, n * k)               # -1 and e take no part
    row_pair = rng.permutation(n * k)
    tw = rng.uniform(0.05, 1.0, (n, k)).astype(np.float32)
    got = swiglu_combine(rows, experts, row_pair, tw, k, wg, wu, wd)
    dec = lambda b: codecs.bf16_bits_to_f32(b).astype(np.float64).tolist()
    for t in range(n):
        terms = [[] for _ in range(d)]
        for j in range(k):
            r = [rr for rr in range(n * k) if row_pair[rr] == t * k + j][0]
            ex = experts[r]
            if not 0 <= ex < e:
                continue
            y = swiglu_brute(dec(rows[r]), dec(wg[ex]), dec(wu[ex]), dec(wd[ex]))
            for i in range(d):
                terms[i].append(float(tw[t, j]) * y[i])
        for i in range(d):
            ref = math.fsum(terms[i])
            mag = math.fsum(abs(v) for v in terms[i])
            assert abs(got[t, i] - ref) <= 1e-3 * mag + 1e-12, (t, i)

"""Pins for the combine oracle (CPU only)."""
import numpy as np
from hypothesis import given, settings, strategies as st

from oracle import codecs, dispatch as od
from oracle.combine import combine_exact_brute, combine_f64
from oracle.route import route_topk


def _f(rows):
    return np.array([[float(v) for v in r] for r in rows], dtype=np.float64)


def test_golden_small(golden):
    g = golden("combine_small.txt")
    y = _f(g["y"]).astype(np.float32)
    dst = np.array([int(v) for v in g["dst_pos"]])
    w = _f(g["w"]).astype(np.float32)
    out = combine_f64(y, dst, w, 2)
    assert np.array_equal(out, _f(g["out"]))
    assert np.array_equal(combine_exact_brute(y, dst, w, 2, "f32"), _f(g["out"]).astype(np.float32))
    bits = np.array([[int(v, 16) for v in r] for r in g["out_bf16"]], dtype=np.uint16)
    assert np.array_equal(combine_exact_brute(y, dst, w, 2, "bf16"), bits)
    assert np.array_equal(codecs.f64_to_bf16_bits(out), bits)
    ty = _f(g["tie.y"]).reshape(2, 1).astype(np.float32)
    tdst = np.array([int(v) for v in g["tie.dst_pos"]])
    for wk, ok in (("tie.w1", "tie.out1_bf16"), ("tie.w2", "tie.out2_bf16")):
        tw = np.array([[float(v) for v in g[wk]]], dtype=np.float32)
        expect = int(g[ok][0], 16)
        assert combine_exact_brute(ty, tdst, tw, 2, "bf16")[0, 0] == expect
        assert codecs.f64_to_bf16_bits(combine_f64(ty, tdst, tw, 2))[0, 0] == expect


@settings(max_examples=40, deadline=None)
@given(st.integers(1, 6), st.integers(1, 4), st.integers(1, 5), st.integers(0, 2**31))
def test_f64_form_matches_exact_brute(n, k, d, seed):
    rng = np.random.default_rng(seed)
    y = rng.standard_normal((n * k, d)).astype(np.float32)
    dst = rng.permutation(n * k)
    w = rng.uniform(-1, 1, (n, k)).astype(np.float32)
    f = combine_f64(y, dst, w, k)
    exact32 = combine_exact_brute(y, dst, w, k, "f32")
    assert np.array_equal(codecs.f64_to_f32(f), exact32)
    exact16 = combine_exact_brute(y, dst, w, k, "bf16")
    # float64 summation error is far below half a bf16 ulp except at exact ties
    assert (np.abs(codecs.f64_to_bf16_bits(f).astype(np.int32) - exact16.astype(np.int32)) <= 1).all()


def test_identity_experts_reproduce_input():
    rng = np.random.default_rng(2)
    n, e, k, d = 64, 32, 8, 48
    x = rng.standard_normal((n, d)).astype(np.float32)
    idx, w = route_topk(rng.standard_normal((n, e)).astype(np.float32), k)
    src, dst, _ = od.permutation(idx, e, 1, True)
    rows = od.gather_rows(x, src, k)
    out = combine_f64(rows, dst, w, k)
    # sum_j w_j = 1 within k fp32 roundings of the weights
    np.testing.assert_allclose(out, x, rtol=2 * k * 2**-24, atol=0)


def test_one_hot_round_trip_is_bit_exact():
    rng = np.random.default_rng(3)
    n, e, k, d = 30, 16, 4, 20
    xb = codecs.f32_to_bf16_bits(rng.standard_normal((n, d)).astype(np.float32))
    idx = np.stack([rng.permutation(e)[:k] for _ in range(n)]).astype(np.int32)
    src, dst, _ = od.permutation(idx, e, 4, False)
    rows = od.gather_rows(xb, src, k)
    for hot in range(k):
        w = np.zeros((n, k), np.float32)
        w[:, hot] = 1.0
        out = combine_f64(codecs.bf16_bits_to_f32(rows), dst, w, k)
        assert np.array_equal(codecs.f64_to_bf16_bits(out), xb)


def test_weight_scaling_is_exact():
    rng = np.random.default_rng(4)
    y = rng.standard_normal((12, 7)).astype(np.float32)
    dst = rng.permutation(12)
    w = rng.uniform(0, 1, (4, 3)).astype(np.float32)
    assert np.array_equal(combine_f64(y, dst, 2 * w, 3), 2 * combine_f64(y, dst, w, 3))


def test_token_subset_matches_full():
    rng = np.random.default_rng(5)
    y = rng.standard_normal((40, 9)).astype(np.float32)
    dst = rng.permutation(40)
    w = rng.uniform(0, 1, (10, 4)).astype(np.float32)
    full = combine_f64(y, dst, w, 4)
    sub = combine_f64(y, dst, w, 4, tokens=[7, 2, 9])
    assert np.array_equal(sub, full[[7, 2, 9]])

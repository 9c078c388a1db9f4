"""Pins for the grouped SwiGLU oracle (CPU only)."""
import numpy as np

from oracle import codecs, dispatch as od
from oracle.swiglu import grouped_swiglu, silu, swiglu_brute, swiglu_rows


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

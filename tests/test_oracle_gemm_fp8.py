"""Pins for the fp8 block-scaled grouped GEMM of the oracle (CPU only)."""
from fractions import Fraction

import numpy as np
import torch

from oracle import codecs
from oracle.gemm_fp8 import (gemm_fp8_brute, gemm_fp8_magnitude, gemm_fp8_rows,
                             grouped_gemm_fp8)


def _codes(rng, shape):
    q = rng.integers(0, 256, shape, dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x30                 # no NaN codes
    return q


def test_closed_form_constant_codes_non_square_block_grid():
    # every code 1.0 (0x38); N = 256 (2 column blocks), K = 384 (3 K blocks), so a
    # transposed scale grid reads out of shape or the wrong block
    r, n, k = 3, 256, 384
    rows = np.full((r, k), 0x38, np.uint8)
    w = np.full((2, n, k), 0x38, np.uint8)
    sx = np.array([[2.0 ** -(p + b) for b in range(3)] for p in range(r)], np.float32)
    sw = np.array([[[2.0 ** (e + 2 * c - b) for b in range(3)] for c in range(2)]
                   for e in range(2)], np.float32)
    experts = np.array([0, 1, 1])
    y = gemm_fp8_rows(rows, sx, experts, w, sw)
    for p in range(r):
        for j in (0, 127, 128, 255):
            want = sum(128 * 2.0 ** -(p + b) * 2.0 ** (experts[p] + 2 * (j // 128) - b)
                       for b in range(3))
            assert y[p, j] == want


def test_matches_exact_rational_brute_force():
    rng = np.random.default_rng(11)
    rows = _codes(rng, (4, 256))
    w = _codes(rng, (2, 128, 256))
    sx = rng.uniform(1e-3, 1e-1, (4, 2)).astype(np.float32)
    sw = rng.uniform(1e-3, 1e-1, (2, 1, 2)).astype(np.float32)
    experts = np.array([1, 0, 1, 0])
    got = gemm_fp8_rows(rows, sx, experts, w, sw)
    mag = gemm_fp8_magnitude(rows, sx, experts, w, sw)
    exact = gemm_fp8_brute(rows, sx, experts, w, sw)
    # float64 rounds each block's scaled term and the running sum: a few units
    # of 2^-53 of the terms' magnitude (the blocks may cancel)
    for p in range(4):
        for j in range(0, 128, 7):
            assert abs(Fraction(float(got[p, j])) - exact[p][j]) <= Fraction(float(mag[p, j])) * Fraction(1, 2 ** 50)


def test_matches_torch_decode_and_matmul():
    rng = np.random.default_rng(12)
    e, n, k = 3, 256, 512
    rows = _codes(rng, (6, k))
    w = _codes(rng, (e, n, k))
    sx = rng.uniform(0.01, 1.0, (6, k // 128)).astype(np.float32)
    sw = rng.uniform(0.01, 1.0, (e, n // 128, k // 128)).astype(np.float32)
    experts = np.array([2, 0, 0, 1, 2, 2])
    dec = lambda a: torch.from_numpy(a).view(torch.float8_e4m3fn).double().numpy()
    xd = dec(rows) * np.repeat(sx.astype(np.float64), 128, axis=1)
    got = gemm_fp8_rows(rows, sx, experts, w, sw)
    for p in range(6):
        wd = dec(w[experts[p]]) * np.repeat(np.repeat(sw[experts[p]].astype(np.float64), 128, 0), 128, 1)
        want = wd @ xd[p]
        assert np.allclose(got[p], want, rtol=1e-12, atol=1e-12 * np.abs(want).max())
    mag = gemm_fp8_magnitude(rows, sx, experts, w, sw)
    assert (mag >= np.abs(got) * (1 - 1e-12)).all()
    # a subset of output columns spread over both 128-column blocks, out of order:
    # each column keeps its own block's weight scale
    cols = np.array([255, 0, 127, 128, 200, 3])
    sub = gemm_fp8_rows(rows, sx, experts, w, sw, cols=cols)
    for p in range(6):
        wd = dec(w[experts[p]]) * np.repeat(np.repeat(sw[experts[p]].astype(np.float64), 128, 0), 128, 1)
        want = (wd @ xd[p])[cols]
        assert np.allclose(sub[p], want, rtol=1e-12, atol=1e-12 * np.abs(want).max())
    assert np.array_equal(gemm_fp8_magnitude(rows, sx, experts, w, sw, cols=cols), mag[:, cols])


def test_ragged_offsets_pick_each_rows_expert():
    rng = np.random.default_rng(13)
    e, n, k = 3, 128, 128
    rows = _codes(rng, (5, k))
    base = _codes(rng, (n, k))
    w = np.stack([base] * e)
    sx = np.ones((5, 1), np.float32)
    sw = np.array([[[1.0]], [[2.0]], [[4.0]]], np.float32)   # expert e scales by 2^e
    bits, y = grouped_gemm_fp8(rows, sx, [0, 2, 2, 5], w, sw)  # expert 1 is empty
    one = gemm_fp8_rows(rows, sx, np.zeros(5, np.int64), w, sw)
    assert np.array_equal(y[:2], one[:2])
    assert np.array_equal(y[2:], 4.0 * one[2:])
    assert np.array_equal(bits, codecs.f64_to_bf16_bits(y))
    bits2, y2 = grouped_gemm_fp8(rows, sx, [0, 1, 1, 3], w, sw)   # rows 3, 4 outside
    assert (y2[3:] == 0).all()

"""Pins for the fp8 identity expert of the oracle (CPU only)."""
from fractions import Fraction

import numpy as np
import torch

from oracle import codecs
from oracle.experts import dequant_rows


def test_exact_codes():
    rows = np.full((2, 128), 0x38, dtype=np.uint8)      # 1.0
    rows[1, :] = 0x7E                                   # 448
    scales = np.array([[0.25], [2.0]], dtype=np.float32)
    y = codecs.bf16_bits_to_f32(dequant_rows(rows, scales))
    assert (y[0] == 0.25).all() and (y[1] == 896.0).all()


def test_matches_torch_decode_and_exact_rounding():
    rng = np.random.default_rng(0)
    rows = rng.integers(0, 256, (3, 256), dtype=np.uint8)
    rows[(rows & 0x7F) == 0x7F] = 0x10                  # no NaN codes
    scales = rng.uniform(1e-3, 1e-1, (3, 2)).astype(np.float32)
    got = dequant_rows(rows, scales)
    ref_q = torch.from_numpy(rows).view(torch.float8_e4m3fn).double().numpy()
    for r in range(3):
        for i in range(256):
            exact = Fraction(float(ref_q[r, i])) * Fraction(float(scales[r, i // 128]))
            want = codecs.fraction_to_bf16_bits(exact)
            if exact == 0 and np.signbit(ref_q[r, i]):
                want = 0x8000                           # -0.0 * s keeps its sign
            assert got[r, i] == want

"""Pins for the oracle's number-format codecs (CPU only)."""
from fractions import Fraction

import numpy as np
import torch

from oracle import codecs
from oracle.swiglu import _bf16_round_py


def test_bf16_decode_all_patterns_vs_torch():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = codecs.bf16_bits_to_f32(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    same = (ours.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def test_f32_to_bf16_rne_vs_torch():
    rng = np.random.default_rng(11)
    vals = np.concatenate([
        rng.standard_normal(200_000).astype(np.float32),
        (rng.standard_normal(50_000) * 1e30).astype(np.float32),
        (rng.standard_normal(50_000) * 1e-39).astype(np.float32),     # subnormals
        rng.integers(0, 2**32, 200_000, dtype=np.uint64).astype(np.uint32).view(np.float32),
        # exact ties: low half 0x8000 with even and odd kept parts
        (np.arange(0x3F800000, 0x3F800000 + 2000 * 0x10000, 0x10000, dtype=np.uint32) | 0x8000).view(np.float32),
        np.array([3.3895314e38, np.float32(np.finfo(np.float32).max), -0.0, 0.0, np.inf, -np.inf], dtype=np.float32),
    ])
    ours = codecs.f32_to_bf16_bits(vals)
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(vals)
    assert (ours[~nan] == ref[~nan]).all()
    assert ((ours[nan] & 0x7FC0) == 0x7FC0).all()


def test_fp8_table_all_patterns_vs_torch():
    bits = np.arange(256, dtype=np.uint8)
    ours = codecs.fp8_bits_to_f64(bits)
    ref = torch.from_numpy(bits).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert ours[0x7E] == 448.0 and np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])
    assert ours[0x01] == 2.0 ** -9


def _frac_round(v: float, frac_bits: int) -> float:
    r = codecs.round_fraction(Fraction(v), frac_bits, -126, 127)
    return float(r)


def test_f64_to_bf16_and_f32_correct_rounding_vs_exact():
    rng = np.random.default_rng(5)
    vals = list(rng.standard_normal(3000) * np.exp(rng.uniform(-40, 40, 3000)))
    # exact bf16 ties and near-ties in float64, where double rounding through
    # float32 with RNE would go wrong
    for base in (1.0, 1.5, 3.25, 1e-3):
        b = float(np.float32(base))
        ulp = 2.0 ** (np.floor(np.log2(abs(b))) - 7)
        vals += [b + ulp / 2, b + ulp / 2 + 2.0 ** -40, b + ulp / 2 - 2.0 ** -40,
                 b + 1.5 * ulp, -(b + ulp / 2)]
    vals = np.array(vals, dtype=np.float64)
    got16 = codecs.bf16_bits_to_f32(codecs.f64_to_bf16_bits(vals)).astype(np.float64)
    got32 = codecs.f64_to_f32(vals).astype(np.float64)
    for v, a, b in zip(vals, got16, got32):
        assert a == _frac_round(v, 7), v
        assert b == _frac_round(v, 23), v
        assert a == _bf16_round_py(v), v        # two independent RNE implementations


def test_fraction_rounding_ties_to_even():
    one = Fraction(1)
    assert codecs.fraction_to_bf16_bits(one + Fraction(1, 256)) == 0x3F80
    assert codecs.fraction_to_bf16_bits(one + Fraction(3, 256)) == 0x3F82
    assert codecs.fraction_to_f32(one + Fraction(1, 2**24)) == np.float32(1.0)
    assert codecs.fraction_to_f32(one + Fraction(3, 2**24)) == np.float32(1.0) + np.float32(2.0 ** -22)

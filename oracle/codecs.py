"""Number-format codecs used by the oracle (test infrastructure only).

* bfloat16: 1 sign, 8 exponent, 7 fraction bits -- the top half of an IEEE
  binary32.  Decoding is a 16-bit shift; encoding rounds to nearest, ties to
  even (RNE), with NaN kept quiet.
* fp8 E4M3FN, the OCP 8-bit floating point format (OFP8 spec, E4M3 variant):
  exponent bias 7, no infinities, S.1111.111 is NaN, largest finite 448,
  subnormals m * 2**-9.  The activations with per-128-element fp32 block
  scales in the segment-major workload use this format.

All functions work on bit patterns held in unsigned integer numpy arrays so
that the oracle never depends on a library's bfloat16 / fp8 type.

Pins (tests/test_oracle_codecs.py): all 2**16 bf16 patterns and all 2**8
fp8 patterns against torch's CPU casts; f32 -> bf16 RNE against torch on
random, tie and overflow cases; f64 -> bf16 / f32 correct rounding against an
exact ``fractions`` rounding on random and tie cases.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


# ----------------------------------------------------------------------------- bf16

def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Decode bfloat16 bit patterns (uint16) to float32 exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (RNE); returns uint16 bit patterns.

    The low 16 bits are dropped with round-half-to-even on the kept part; a
    carry out of the fraction correctly bumps the exponent (up to infinity).
    NaN inputs become a quiet NaN with the same sign.
    """
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint32)
    nan = np.isnan(f)
    if nan.any():
        sign = (u >> np.uint64(16)).astype(np.uint32) & np.uint32(0x8000)
        rounded = np.where(nan, sign | np.uint32(0x7FC0), rounded)
    return rounded.astype(np.uint16)


def _f64_to_f32_round_to_odd(x: np.ndarray) -> np.ndarray:
    """float64 -> float32 rounding to odd: truncate toward zero, then set the
    last bit if anything was lost.  Rounding the result once more to any
    format with at least two fewer fraction bits gives the correctly rounded
    value of ``x`` in that format (Boldo & Melquiond, "When double rounding is
    odd", 2005)."""
    x = np.asarray(x, dtype=np.float64)
    r = x.astype(np.float32)                     # RNE
    over = np.abs(r.astype(np.float64)) > np.abs(x)
    r = np.where(over, np.nextafter(r, np.float32(0)), r)   # toward zero
    inexact = r.astype(np.float64) != x
    bits = r.view(np.uint32) | inexact.astype(np.uint32)
    return np.where(np.isfinite(x), bits.view(np.float32), x.astype(np.float32))


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Correctly rounded (RNE) float64 -> bfloat16 bit patterns."""
    return f32_to_bf16_bits(_f64_to_f32_round_to_odd(x))


def f64_to_f32(x: np.ndarray) -> np.ndarray:
    """Correctly rounded (RNE) float64 -> float32 (numpy's own cast)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


# ----------------------------------------------------------------------------- fp8

def fp8_e4m3fn_table() -> np.ndarray:
    """float64 value of every E4M3FN bit pattern 0..255 (NaN for S.1111.111).

    Built from the format definition: value = (-1)^s * 2^(e-7) * (1 + m/8) for
    exponent field e in 1..15, and (-1)^s * 2^-6 * (m/8) for e == 0.
    """
    out = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = (code >> 7) & 1
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            v = float("nan")
        elif e == 0:
            v = (m / 8.0) * 2.0 ** (1 - 7)
        else:
            v = (1.0 + m / 8.0) * 2.0 ** (e - 7)
        out[code] = -v if s else v
    return out


_FP8_TABLE = fp8_e4m3fn_table()


def fp8_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode E4M3FN bit patterns (uint8) to float64 exactly."""
    return _FP8_TABLE[np.asarray(bits, dtype=np.uint8)]


# ----------------------------------------------------------------------------- exact rounding

def round_fraction(v: Fraction, frac_bits: int, emin: int, emax: int) -> Fraction:
    """Round an exact rational to the nearest value of a binary floating-point
    format with ``frac_bits`` fraction bits, minimum normal exponent ``emin``
    and maximum exponent ``emax`` (ties to even; overflow -> +-inf as a float).

    binary32: (23, -126, 127); bfloat16: (7, -126, 127).
    Used by the brute-force tier to round exact sums once.
    """
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)                       # subnormal spacing below emin
    ulp = Fraction(2) ** (e - frac_bits)
    q, r = divmod(a, ulp)                  # a = q*ulp + r, 0 <= r < ulp
    q = int(q)
    if r * 2 > ulp or (r * 2 == ulp and q % 2 == 1):
        q += 1
    res = q * ulp
    if res >= Fraction(2) ** (emax + 1):
        return Fraction(sign) * Fraction(10) ** 400   # stands for infinity
    return sign * res


def fraction_to_f32(v: Fraction) -> np.float32:
    r = round_fraction(v, 23, -126, 127)
    if abs(r) > Fraction(10) ** 300:
        return np.float32(np.inf if r > 0 else -np.inf)
    return np.float32(float(r))            # exact: r is a binary32 value


def fraction_to_bf16_bits(v: Fraction) -> int:
    r = round_fraction(v, 7, -126, 127)
    if abs(r) > Fraction(10) ** 300:
        f = np.float32(np.inf if r > 0 else -np.inf)
    else:
        f = np.float32(float(r))           # exact: r is a bf16 value
    return int(np.array([f], dtype=np.float32).view(np.uint32)[0] >> 16)

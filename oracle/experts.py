"""Identity expert for the fp8 payload (test infrastructure only).

The segment-major workload carries fp8 E4M3FN activations with one float32
scale per 128 elements of a row; "One-Sided Expert-Parallel All-to-All ...
over NVLink" (abstract) keeps dispatch agnostic to that format, so the
expert side is where it is undone.  With identity experts the expert output
of row p is its dequantised value, rounded once to bfloat16:

    y[p, i] = bf16( value(rows[p, i]) * row_scales[p, i // 128] )

The product of an E4M3 value (4 significant bits) and a float32 scale (24)
is exact in float64, so this is one correct rounding.

Pins (tests/test_oracle_experts.py): codes 0x38 (1.0) and 0x7E (448) with
power-of-two scales decode exactly; the result equals torch's CPU float8 ->
float32 cast times the scale, rounded by an exact Fraction rounding.
"""
from __future__ import annotations

import numpy as np

from .codecs import f64_to_bf16_bits, fp8_bits_to_f64


def dequant_rows(rows_fp8: np.ndarray, row_scales: np.ndarray, block: int = 128) -> np.ndarray:
    q = fp8_bits_to_f64(rows_fp8)
    n, d = q.shape
    s = np.repeat(np.asarray(row_scales, dtype=np.float32).astype(np.float64), block, axis=1)
    return f64_to_bf16_bits(q * s[:, :d])
